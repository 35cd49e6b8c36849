// Host runtime behind the C ABI in include/kva.h: config validation, weight
// conversion and repacking, device memory, and the launch sequence of one
// projection (the hot path).
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kva.h"
#include "kva_internal.h"

using namespace kva;

namespace {

thread_local std::string g_last_error;

kva_status fail(kva_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

#define HIP_TRY(expr)                                                                   \
    do {                                                                                \
        hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess)                                                           \
            return fail(e_ == hipErrorOutOfMemory ? KVA_ERR_OOM : KVA_ERR_HIP, "%s: %s (%s:%d)", \
                        #expr, hipGetErrorString(e_), __FILE__, __LINE__);              \
    } while (0)

// Contexts of at most this many tokens per call run every trunk GEMM on the
// skinny kernel (K split over the waves of a workgroup; the N = d GEMMs
// also over kSkinnySplits workgroups, folded like the tiled split-K).
constexpr int kSkinnyTokens = 32;
constexpr int kSkinnySplits = 4;   // split-K of their N = d GEMMs across workgroups

// Contexts of more than this many tokens per call hold q8_0 / q4_0 weights
// expanded to fp16 (the values the in-register dequantisation forms, so the
// same bits): at those sizes the GEMMs are bound by MFMA issue and power,
// not by weight bytes, and the conversion's VALU work cost 14-19% of the
// head GEMM; smaller contexts keep the code and scale planes (half the
// bytes) for their weight-bandwidth-bound calls.
constexpr int kExpandTokens = 256;

// Split count of the GEMMs whose N is the trunk width (input, O, down): with
// only d = 2560-3072 columns they fill too few workgroups at 1024 tokens.
// Fixed per context (from d and max_tokens, never from a call's token count):
// a row's reduction order, hence its bits, must not depend on the call's
// size.  Three K-ranges when a context with 16-bit trunk weights takes at
// most one 1024-token ubatch per call and the three ranges of its 256x128
// tiles still fit one round over 256 CUs (d <= 2688); two otherwise (more
// partials to fold cost more than they gain once the tiles fill the device).
// Contexts of at most 128 tokens per call (one 128-row tile) read every
// weight once per call and have few tiles: eight K-ranges, so that the
// narrow GEMMs stream their weights from 8x as many workgroups (contexts of
// at most kSkinnyTokens take kSkinnySplits on the skinny kernel).
inline int split_narrow(int64_t d, int64_t max_tokens, bool f16_trunk) {
    if (max_tokens <= 128) return 8;
    return (f16_trunk && max_tokens <= 1024 && d % 128 == 0 && 4 * (d / 128) * 3 <= 256) ? 3 : 2;
}

#define KVA_TRY(expr)                    \
    do {                                 \
        kva_status s_ = (expr);          \
        if (s_ != KVA_OK) return s_;     \
    } while (0)

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// ------------------------------------------------------------------ host number formats

float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

float f16_bits_to_f32(uint16_t h) {
    const uint32_t sign = (uint32_t)(h & 0x8000u) << 16, e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    uint32_t u;
    if (e == 0x1Fu) u = sign | 0x7F800000u | (m << 13);
    else if (e != 0) u = sign | ((e + 112u) << 23) | (m << 13);
    else {
        float f = (float)m * 5.9604644775390625e-8f;     // m * 2^-24, exact
        return (h & 0x8000u) ? -f : f;
    }
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// A q8_0 / q4_0 block whose fp16 weights d * code (the GEMMs' operands,
// d * code rounded once to fp16) would not all be finite: a non-finite
// scale, or |d| * max|code| at or past 65520, which rounds to infinity.
bool quant_block_out_of_range(uint16_t d_bits, int max_abs_code) {
    const float d = f16_bits_to_f32(d_bits);
    return !std::isfinite(d) || std::fabs(d) * (float)max_abs_code >= 65520.0f;
}

// fp32 -> fp16, round to nearest even.  Sets *overflow when a finite input
// rounds to infinity.
uint16_t f32_to_f16(float f, bool* overflow) {
    uint32_t x;
    std::memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
    if (ax >= 0x477FF000u) {            // >= 65520: rounds past 65504
        *overflow = true;
        return (uint16_t)(sign | 0x7C00u);
    }
    if (ax >= 0x38800000u) {            // >= 2^-14: normal fp16
        const uint32_t mant = ax & 0x7FFFFFu;
        uint32_t h = ((((ax >> 23) - 127u + 15u)) << 10) | (mant >> 13);
        const uint32_t rem = mant & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
        return (uint16_t)(sign | h);
    }
    if (ax <= 0x33000000u) return (uint16_t)sign;   // <= 2^-25 rounds to zero
    const uint32_t mant = (ax & 0x7FFFFFu) | 0x800000u;
    const int shift = 126 - (int)(ax >> 23);       // value / 2^-24 = mant >> shift
    uint32_t h = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (h & 1u))) ++h;
    return (uint16_t)(sign | h);
}

uint16_t f32_to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

float load_f32(const void* src, int dtype, int64_t i) {
    if (dtype == KVA_DTYPE_F32) return static_cast<const float*>(src)[i];
    return bf16_to_f32(static_cast<const uint16_t*>(src)[i]);
}

// ------------------------------------------------------------------ head packing

struct HeadPlan {
    int64_t n_pad = 0;
    int32_t tail_start = 0;
    int32_t kv_tiles = 0;                        // leading tiles that belong to KV heads
    std::vector<int32_t> kv_heads;               // KV heads in head order
    std::vector<int32_t> tile_head, tile_col0;   // per kHeadTileN tile
    std::vector<int32_t> tail_head, tail_col;    // per tail column
    std::vector<int32_t> col_head, col_index;    // per packed column
};

// A full-attention head whose output is k | v of kKvHeads heads of kKvHeadDim:
// the fused KV epilogue can take it.
bool is_kv_head(const kva_head_desc& h) {
    return h.kind == KVA_HEAD_ATTN && h.out_dim == 2 * kKvHeads * kKvHeadDim;
}

HeadPlan plan_heads(const kva_config& c) {
    HeadPlan p;
    // KV heads first, so their tiles always run as whole 256-column tiles
    for (int i = 0; i < c.n_out_heads; ++i) {
        if (!is_kv_head(c.out_heads[i])) continue;
        p.kv_heads.push_back(i);
        for (int t = 0; t < c.out_heads[i].out_dim / kHeadTileN; ++t) {
            p.tile_head.push_back(i);
            p.tile_col0.push_back(t * kHeadTileN);
        }
    }
    p.kv_tiles = (int32_t)p.tile_head.size();
    for (int i = 0; i < c.n_out_heads; ++i) {
        if (is_kv_head(c.out_heads[i])) continue;
        const int full = c.out_heads[i].out_dim / kHeadTileN;
        for (int t = 0; t < full; ++t) {
            p.tile_head.push_back(i);
            p.tile_col0.push_back(t * kHeadTileN);
        }
    }
    p.tail_start = (int32_t)p.tile_head.size() * kHeadTileN;
    for (int i = 0; i < c.n_out_heads; ++i) {
        const int od = c.out_heads[i].out_dim;
        for (int col = od / kHeadTileN * kHeadTileN; col < od; ++col) {
            p.tail_head.push_back(i);
            p.tail_col.push_back(col);
        }
    }
    const int64_t tail_pad = round_up((int64_t)p.tail_head.size(), kHeadTileN);
    p.tail_head.resize(tail_pad, -1);
    p.tail_col.resize(tail_pad, 0);
    for (int64_t t = 0; t < tail_pad / kHeadTileN; ++t) {
        p.tile_head.push_back(-1);
        p.tile_col0.push_back(0);
    }
    if (p.tail_head.empty()) {   // keep the device arrays non-empty
        p.tail_head.push_back(-1);
        p.tail_col.push_back(0);
    }
    p.n_pad = (int64_t)p.tile_head.size() * kHeadTileN;
    p.col_head.resize(p.n_pad);
    p.col_index.resize(p.n_pad);
    for (int64_t c2 = 0; c2 < p.tail_start; ++c2) {
        p.col_head[c2] = p.tile_head[c2 / kHeadTileN];
        p.col_index[c2] = p.tile_col0[c2 / kHeadTileN] + (int32_t)(c2 % kHeadTileN);
    }
    for (int64_t c2 = p.tail_start; c2 < p.n_pad; ++c2) {
        p.col_head[c2] = p.tail_head[c2 - p.tail_start];
        p.col_index[c2] = p.tail_col[c2 - p.tail_start];
    }
    return p;
}

}  // namespace

// ------------------------------------------------------------------ context

struct kva_ctx {
    kva_config cfg{};
    std::vector<kva_head_desc> heads;
    int device = 0;
    int n_cu = 0;                  // compute units of the device (head GEMM round size)
    std::vector<void*> allocs;
    std::vector<std::pair<void*, size_t>> scratch_regions;   // activation scratch (kva_debug_poison_scratch)
    uint64_t weight_bytes = 0, scratch_bytes = 0;

    // weights (device).  A weight is either 16-bit values w16 (fp16 trunk,
    // bf16 heads; tiled as in tiled32_index) or, for q8_0, int8 codes q and
    // fp16 scales sc (tiled as in q8_code_chunk / q8_scale_index).  Every
    // GEMM activation operand is in the tiled32 layout (its producer writes
    // it so).
    struct DevW {
        uint16_t* w16 = nullptr;
        int8_t* q = nullptr;
        uint16_t* sc = nullptr;
    };
    bool q8 = false;               // block-quantised weights (q8_0 or q4_0): fp16 activations
    bool q4 = false;               // ... and they are q4_0
    // GEMM operands: fp16 trunk / bf16 heads for fp32 and bf16 weights;
    // the code and scale planes for q8_0 / q4_0, or, in contexts of more than
    // kExpandTokens tokens per call, those weights expanded to fp16 at create
    GemmOperand trunk_opd = OPD_F16, head_opd = OPD_BF16;
    DevW w_in;
    float* g_in = nullptr;
    float* g_out = nullptr;
    struct Blk {
        float* g_attn = nullptr;
        float* g_ffn = nullptr;
        DevW wqkv;   // [pad(3 hd)][d]: rows wq | wk | wv
        DevW wo;     // [pad(d)][hd]
        DevW wgu;    // [pad(2 F)][d]: per 64 rows, 32 gate rows then the matching 32 up rows
        DevW wd;     // [pad(d)][F]
    };
    std::vector<Blk> blk;
    DevW w_heads;                  // [n_pad][d], packed column order
    float* b_heads = nullptr;      // [n_pad]
    int32_t* tile_head = nullptr;
    int32_t* tile_col0 = nullptr;
    int32_t* tail_head = nullptr;
    int32_t* tail_col = nullptr;
    int64_t n_pad_heads = 0;
    int32_t tail_start = 0;
    bool map_only = false;            // a single-map context (kva_map_create): heads on the raw input
    int32_t kv_tiles = 0;             // leading packed tiles of the KV heads
    std::vector<int32_t> kv_heads;    // heads the fused KV epilogue takes, in head order

    // scratch (device), rows padded to kRowPad
    int64_t m_alloc = 0;
    uint16_t* u16 = nullptr;    // [m][n_in]   fp16 normed input (skinny contexts only)
    float* ss_in = nullptr;     // [n_split][m] input rows' sums of squares per K split (EPI_INPUT)
    float* h = nullptr;         // [m][d]      fp32 residual stream
    uint16_t* a16 = nullptr;    // [m][d]      fp16 normed activations
    uint16_t* qk16 = nullptr;   // [m][2 hd]   fp16 Q | K
    uint16_t* vt16 = nullptr;   // [hd][m]     fp16 V transposed
    uint16_t* o16 = nullptr;    // [m][hd]     fp16 attention output
    uint16_t* act16 = nullptr;  // [m][F]      fp16 SwiGLU output
    uint16_t* z16 = nullptr;    // [m][d]      final-normed trunk state: bf16 (fp16 for q8_0)
    float* ws = nullptr;        // [n_split][m][d] split-K partials of the N = d GEMMs
    int n_split = 2;            // split count of the N = d GEMMs (split_narrow)
    bool skinny = false;        // every trunk GEMM on the skinny kernel (max_tokens <= kSkinnyTokens)

    kva_stats stats{};

    // kva_profile_*: event pairs recorded around the launches of selected stages
    uint32_t prof_mask = 0;
    struct Rec {
        int stage;
        hipEvent_t a, b;
    };
    std::vector<Rec> prof_pending;
    std::vector<hipEvent_t> prof_free;
    kva_stage_time prof_acc[KVA_N_STAGES]{};

    hipEvent_t take_event() {
        if (!prof_free.empty()) {
            hipEvent_t e = prof_free.back();
            prof_free.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }

    template <class T>
    hipError_t alloc(T** p, size_t bytes, bool weight) {
        void* q = nullptr;
        hipError_t e = hipMalloc(&q, bytes);
        if (e != hipSuccess) return e;
        allocs.push_back(q);
        (weight ? weight_bytes : scratch_bytes) += bytes;
        if (!weight) scratch_regions.push_back({q, bytes});
        *p = static_cast<T*>(q);
        return hipSuccess;
    }
    ~kva_ctx() {
        for (Rec& r : prof_pending) {
            (void)hipEventDestroy(r.a);
            (void)hipEventDestroy(r.b);
        }
        for (hipEvent_t e : prof_free) (void)hipEventDestroy(e);
        for (void* p : allocs) (void)hipFree(p);
    }
};

namespace {

kva_status validate(const kva_config* c) {
    if (!c) return fail(KVA_ERR_ARG, "config is NULL");
    if (c->n_in <= 0 || c->d_model <= 0 || c->n_blocks <= 0 || c->n_heads <= 0 ||
        c->head_dim <= 0 || c->d_ffn <= 0 || c->attn_block <= 0 || c->max_tokens <= 0)
        return fail(KVA_ERR_SHAPE, "all dimensions must be positive");
    if (c->head_dim != 128) return fail(KVA_ERR_SHAPE, "head_dim must be 128 (got %d)", c->head_dim);
    if ((int64_t)c->n_heads * c->head_dim != c->d_model)
        return fail(KVA_ERR_SHAPE, "n_heads*head_dim (%d) must equal d_model (%d)",
                    c->n_heads * c->head_dim, c->d_model);
    if (c->n_in % 64 || c->d_model % 64 || c->d_ffn % 64)
        return fail(KVA_ERR_SHAPE, "n_in, d_model and d_ffn must be multiples of 64");
    if (c->attn_block % 64) return fail(KVA_ERR_SHAPE, "attn_block must be a multiple of 64");
    if (c->n_blocks > 64) return fail(KVA_ERR_SHAPE, "at most 64 transformer blocks");
    if (c->max_tokens > (1 << 24)) return fail(KVA_ERR_SHAPE, "max_tokens above 2^24");
    if (!(c->eps >= 0.0f) || !std::isfinite(c->eps)) return fail(KVA_ERR_ARG, "eps must be finite and >= 0");
    if (c->weight_dtype != KVA_DTYPE_F32 && c->weight_dtype != KVA_DTYPE_BF16 &&
        c->weight_dtype != KVA_DTYPE_Q8_0 && c->weight_dtype != KVA_DTYPE_Q4_0)
        return fail(KVA_ERR_DTYPE, "unknown weight dtype %d", c->weight_dtype);
    if (c->has_head_bias != 0 && c->has_head_bias != 1) return fail(KVA_ERR_ARG, "has_head_bias must be 0 or 1");
    if (c->n_out_heads < 1 || c->n_out_heads > kMaxHeads)
        return fail(KVA_ERR_SHAPE, "n_out_heads must be in [1, %d]", kMaxHeads);
    if (!c->out_heads) return fail(KVA_ERR_ARG, "out_heads is NULL");
    for (int i = 0; i < c->n_out_heads; ++i) {
        const kva_head_desc& h = c->out_heads[i];
        if (h.out_dim <= 0 || h.out_dim > (1 << 20)) return fail(KVA_ERR_SHAPE, "head %d: bad out_dim %d", i, h.out_dim);
        if (h.kind < KVA_HEAD_DELTANET || h.kind > KVA_HEAD_DRAFT) return fail(KVA_ERR_ARG, "head %d: bad kind", i);
    }
    return KVA_OK;
}

// Converts a [rows][cols] weight (fp32 or bf16) to fp16 at dst.
kva_status to_f16_rows(const void* src, int dtype, int64_t rows, int64_t cols, uint16_t* dst,
                       const char* name) {
    if (!src) return fail(KVA_ERR_ARG, "weight %s is NULL", name);
    bool ovf = false;
    const int64_t n = rows * cols;
    for (int64_t i = 0; i < n; ++i) dst[i] = f32_to_f16(load_f32(src, dtype, i), &ovf);
    if (ovf) return fail(KVA_ERR_RANGE, "weight %s has values outside the fp16 range", name);
    return KVA_OK;
}

kva_status upload(kva_ctx* ctx, void* dst, const void* src, size_t bytes) {
    HIP_TRY(hipMemcpy(dst, src, bytes, hipMemcpyHostToDevice));
    return KVA_OK;
}

// One destination row of a packed weight: row `row` of source tensor `src`,
// or a zero row when src is NULL (padding).
struct RowSrc {
    const void* src;
    int64_t row;
};

// Target layouts on the device.
enum PackTarget { PACK_F16_T32 = 0, PACK_BF16_T32 = 1, PACK_Q8 = 2, PACK_Q4 = 3 };

// A weight in its device layout, still on the host: 16-bit values w16 in the
// tiled32_index layout, or int8/4-bit codes q and fp16 scales sc (q8_0 /
// q4_0 planes, q8_code_chunk / q4_code_chunk and q8_scale_index layouts).
struct HostPacked {
    std::vector<uint16_t> w16;
    std::vector<uint8_t> q;
    std::vector<uint16_t> sc;
};

// Packs rows (each K wide, stored in `dtype`) into the compute layout on the
// host: fp16 or bf16 values in the tiled layout of tiled32_index (32-wide
// slabs), or for q8_0 / q4_0 the blocks split losslessly into a code plane
// and an fp16 scale plane, tiled the same way.  Host memory only.
kva_status pack_host(int dtype, int64_t K, const std::vector<RowSrc>& rows, PackTarget target, HostPacked* out,
                     const char* name) {
    const int64_t n = (int64_t)rows.size();
    for (const RowSrc& r : rows)
        if (!r.src && r.row >= 0) return fail(KVA_ERR_ARG, "weight %s is NULL", name);
    if (n % kWeightTileRows || K % 32 || K <= 0) return fail(KVA_ERR_SHAPE, "weight %s: bad padding", name);
    if (target == PACK_Q4) {
        if (dtype != KVA_DTYPE_Q4_0) return fail(KVA_ERR_DTYPE, "q4_0 layout needs q4_0 weights (%s)", name);
        const int64_t nb = K / 32;
        std::vector<uint8_t>& q = out->q;
        std::vector<uint16_t>& sc = out->sc;
        q.assign((size_t)(n * K / 2), 0x88);   // padding rows: codes 8 (and scale 0)
        sc.assign((size_t)(n * nb), 0);
        for (int64_t r = 0; r < n; ++r) {
            if (!rows[r].src) continue;
            const uint8_t* blk = static_cast<const uint8_t*>(rows[r].src) + rows[r].row * nb * 18;
            for (int64_t b = 0; b < nb; ++b) {
                const uint8_t* qs = blk + b * 18 + 2;
                const uint16_t d_bits = (uint16_t)(blk[b * 18] | (blk[b * 18 + 1] << 8));
                int mx = 0;
                for (int j = 0; j < 16; ++j) {
                    const int lo = std::abs((qs[j] & 0xF) - 8), hi = std::abs((qs[j] >> 4) - 8);
                    mx = std::max(mx, std::max(lo, hi));
                }
                if (quant_block_out_of_range(d_bits, mx))
                    return fail(KVA_ERR_RANGE, "weight %s: q4_0 block (row %lld, block %lld) has a scale whose "
                                "weights d*(n-8) are not finite in fp16", name, (long long)rows[r].row, (long long)b);
                sc[(size_t)q8_scale_index(r, b, K)] = d_bits;
                for (int64_t c = 0; c < 4; ++c) {       // 8 inputs of the block per chunk
                    uint8_t nn[8];
                    for (int e = 0; e < 8; ++e) {
                        const int k = (int)(8 * c) + e;
                        nn[e] = k < 16 ? (qs[k] & 0xF) : (qs[k - 16] >> 4);
                    }
                    const uint32_t w = q4_chunk_pack(nn);
                    std::memcpy(&q[(size_t)q4_code_chunk(r, b * 32 + 8 * c, K)], &w, 4);
                }
            }
        }
        return KVA_OK;
    }
    if (target == PACK_Q8) {
        if (dtype != KVA_DTYPE_Q8_0) return fail(KVA_ERR_DTYPE, "q8_0 layout needs q8_0 weights (%s)", name);
        const int64_t nb = K / 32;
        std::vector<uint8_t>& q = out->q;
        std::vector<uint16_t>& sc = out->sc;
        q.assign((size_t)(n * K), 0);
        sc.assign((size_t)(n * nb), 0);
        for (int64_t r = 0; r < n; ++r) {
            if (!rows[r].src) continue;
            const uint8_t* blk = static_cast<const uint8_t*>(rows[r].src) + rows[r].row * nb * 34;
            for (int64_t b = 0; b < nb; ++b) {
                const uint16_t d_bits = (uint16_t)(blk[b * 34] | (blk[b * 34 + 1] << 8));
                const int8_t* codes = reinterpret_cast<const int8_t*>(blk + b * 34 + 2);
                int mx = 0;
                for (int j = 0; j < 32; ++j) mx = std::max(mx, std::abs((int)codes[j]));
                if (quant_block_out_of_range(d_bits, mx))
                    return fail(KVA_ERR_RANGE, "weight %s: q8_0 block (row %lld, block %lld) has a scale whose "
                                "weights d*q are not finite in fp16", name, (long long)rows[r].row, (long long)b);
                sc[(size_t)q8_scale_index(r, b, K)] = d_bits;
                for (int64_t c = 0; c < 32; c += 8) {   // 8 consecutive codes form one chunk
                    uint32_t w[2];
                    q8_chunk_pack(codes + c, &w[0], &w[1]);
                    std::memcpy(&q[(size_t)q8_code_chunk(r, b * 32 + c, K)], w, 8);
                }
            }
        }
        return KVA_OK;
    }
    const bool quant = dtype == KVA_DTYPE_Q8_0 || dtype == KVA_DTYPE_Q4_0;
    if (dtype != KVA_DTYPE_F32 && dtype != KVA_DTYPE_BF16 && !(quant && target == PACK_F16_T32))
        return fail(KVA_ERR_DTYPE, "16-bit layout needs fp32 or bf16 weights, or q8_0 / q4_0 for fp16 (%s)", name);
    std::vector<uint16_t> w((size_t)(n * K), 0);
    bool ovf = false;
    for (int64_t r = 0; r < n; ++r) {
        if (!rows[r].src) continue;
        uint16_t* dst = &w[(size_t)(r * K)];
        const int64_t base = rows[r].row * K;
        if (quant) {
            // q8_0 / q4_0 blocks expanded to the fp16 weights the in-register
            // dequantisation forms: d * code is exact in fp32 (11 x 8 bits),
            // rounded once to fp16, so the GEMM multiplies the same values
            const bool is4 = dtype == KVA_DTYPE_Q4_0;
            const int bb = is4 ? 18 : 34;
            const uint8_t* blk = static_cast<const uint8_t*>(rows[r].src) + rows[r].row * (K / 32) * bb;
            for (int64_t b = 0; b < K / 32; ++b) {
                const uint8_t* p = blk + b * bb;
                const uint16_t d_bits = (uint16_t)(p[0] | (p[1] << 8));
                int mx = 0;
                int code[32];
                for (int j = 0; j < 32; ++j) {
                    code[j] = is4 ? (j < 16 ? (p[2 + j] & 0xF) : (p[2 + j - 16] >> 4)) - 8 : (int)(int8_t)p[2 + j];
                    mx = std::max(mx, std::abs(code[j]));
                }
                if (quant_block_out_of_range(d_bits, mx))
                    return fail(KVA_ERR_RANGE, "weight %s: %s block (row %lld, block %lld) has a scale whose "
                                "weights are not finite in fp16", name, is4 ? "q4_0" : "q8_0",
                                (long long)rows[r].row, (long long)b);
                const float d = f16_bits_to_f32(d_bits);
                for (int j = 0; j < 32; ++j) dst[b * 32 + j] = f32_to_f16(d * (float)code[j], &ovf);
            }
        } else if (target == PACK_BF16_T32 && dtype == KVA_DTYPE_BF16) {
            std::memcpy(dst, static_cast<const uint16_t*>(rows[r].src) + base, (size_t)K * 2);
        } else if (target == PACK_BF16_T32) {
            for (int64_t k = 0; k < K; ++k) dst[k] = f32_to_bf16(static_cast<const float*>(rows[r].src)[base + k]);
        } else {
            for (int64_t k = 0; k < K; ++k) dst[k] = f32_to_f16(load_f32(rows[r].src, dtype, base + k), &ovf);
        }
    }
    if (ovf) return fail(KVA_ERR_RANGE, "weight %s has values outside the fp16 range", name);
    std::vector<uint16_t>& t = out->w16;
    t.assign(w.size(), 0);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t k = 0; k < K; k += 8)    // 8 consecutive K-values stay together
            std::memcpy(&t[(size_t)tiled32_index(r, k, K)], &w[(size_t)(r * K + k)], 16);
    return KVA_OK;
}

// pack_host, then upload into memory the context owns.
kva_status pack_weight(kva_ctx* ctx, int dtype, int64_t K, const std::vector<RowSrc>& rows,
                       PackTarget target, kva_ctx::DevW* out, const char* name) {
    HostPacked hp;
    KVA_TRY(pack_host(dtype, K, rows, target, &hp, name));
    if (target == PACK_Q8 || target == PACK_Q4) {
        HIP_TRY(ctx->alloc(&out->q, hp.q.size(), true));
        HIP_TRY(ctx->alloc(&out->sc, hp.sc.size() * 2, true));
        KVA_TRY(upload(ctx, out->q, hp.q.data(), hp.q.size()));
        return upload(ctx, out->sc, hp.sc.data(), hp.sc.size() * 2);
    }
    HIP_TRY(ctx->alloc(&out->w16, hp.w16.size() * 2, true));
    return upload(ctx, out->w16, hp.w16.data(), hp.w16.size() * 2);
}

// Rows [0, n) of one tensor, then zero rows up to a multiple of kColPad.
void add_rows(std::vector<RowSrc>& v, const void* src, int64_t n) {
    for (int64_t r = 0; r < n; ++r) v.push_back({src, r});
}
void pad_rows(std::vector<RowSrc>& v) {
    while (v.size() % kColPad) v.push_back({nullptr, -1});
}

// The head weights and biases of config c (inputs d wide) in packed column
// order (plan_heads), with the device tables of the packing.
kva_status pack_heads(kva_ctx* ctx, const kva_config& c, const void* const* head_w, const float* const* head_b,
                      int64_t d, PackTarget head_t) {
    const int dt = c.weight_dtype;
    if (!head_w) return fail(KVA_ERR_ARG, "head_w is NULL");
    if (c.has_head_bias && !head_b) return fail(KVA_ERR_ARG, "head_b is NULL but has_head_bias is set");
    for (int i = 0; i < c.n_out_heads; ++i) {
        if (!head_w[i]) return fail(KVA_ERR_ARG, "head_w[%d] is NULL", i);
        if (c.has_head_bias && !head_b[i]) return fail(KVA_ERR_ARG, "head_b[%d] is NULL", i);
    }
    HeadPlan plan = plan_heads(c);
    ctx->n_pad_heads = plan.n_pad;
    ctx->tail_start = plan.tail_start;
    ctx->kv_tiles = plan.kv_tiles;
    ctx->kv_heads = plan.kv_heads;
    {
        std::vector<RowSrc> rows((size_t)plan.n_pad);
        std::vector<float> bias((size_t)plan.n_pad, 0.0f);
        for (int64_t col = 0; col < plan.n_pad; ++col) {
            const int hh = plan.col_head[col];
            if (hh < 0) {
                rows[col] = {nullptr, -1};
                continue;
            }
            rows[col] = {head_w[hh], plan.col_index[col]};
            if (c.has_head_bias) bias[col] = head_b[hh][plan.col_index[col]];
        }
        KVA_TRY(pack_weight(ctx, dt, d, rows, head_t, &ctx->w_heads, "heads"));
        float* bb = nullptr;
        HIP_TRY(ctx->alloc(&bb, (size_t)plan.n_pad * 4, true));
        KVA_TRY(upload(ctx, bb, bias.data(), (size_t)plan.n_pad * 4));
        ctx->b_heads = c.has_head_bias ? bb : nullptr;
    }
    auto puti = [&](int32_t** dstp, const std::vector<int32_t>& v) -> kva_status {
        HIP_TRY(ctx->alloc(dstp, v.size() * 4, true));
        return upload(ctx, *dstp, v.data(), v.size() * 4);
    };
    KVA_TRY(puti(&ctx->tile_head, plan.tile_head));
    KVA_TRY(puti(&ctx->tile_col0, plan.tile_col0));
    KVA_TRY(puti(&ctx->tail_head, plan.tail_head));
    KVA_TRY(puti(&ctx->tail_col, plan.tail_col));
    return KVA_OK;
}

kva_status create_impl(const kva_config* cfg, const kva_weights* w, int device, kva_ctx* ctx) {
    const kva_config& c = *cfg;
    const int dt = c.weight_dtype;
    const bool q4 = dt == KVA_DTYPE_Q4_0;
    const bool q8 = dt == KVA_DTYPE_Q8_0 || q4;
    if (q8 && (c.n_in % 32 || c.d_model % 32 || c.d_ffn % 32))
        return fail(KVA_ERR_SHAPE, "q8_0 / q4_0 need every Linear input width to be a multiple of 32");
    const int64_t d = c.d_model, F = c.d_ffn, n_in = c.n_in;
    const int64_t hd = (int64_t)c.n_heads * c.head_dim;
    HIP_TRY(hipSetDevice(device));
    ctx->device = device;
    HIP_TRY(hipDeviceGetAttribute(&ctx->n_cu, hipDeviceAttributeMultiprocessorCount, device));
    ctx->q8 = q8;
    ctx->q4 = q4;
    const bool expand = q8 && c.max_tokens > kExpandTokens;
    const PackTarget trunk_t = expand ? PACK_F16_T32 : q4 ? PACK_Q4 : q8 ? PACK_Q8 : PACK_F16_T32;
    const PackTarget head_t = expand ? PACK_F16_T32 : q4 ? PACK_Q4 : q8 ? PACK_Q8 : PACK_BF16_T32;
    ctx->trunk_opd = expand ? OPD_F16 : q4 ? OPD_Q4 : q8 ? OPD_Q8 : OPD_F16;
    ctx->head_opd = expand ? OPD_F16 : q4 ? OPD_Q4 : q8 ? OPD_Q8 : OPD_BF16;

    auto putf = [&](float** dstp, const float* src, int64_t n, const char* name) -> kva_status {
        if (!src) return fail(KVA_ERR_ARG, "gain %s is NULL", name);
        HIP_TRY(ctx->alloc(dstp, (size_t)n * 4, true));
        return upload(ctx, *dstp, src, (size_t)n * 4);
    };

    // -------- trunk
    KVA_TRY(putf(&ctx->g_in, w->in_norm, n_in, "in_norm"));
    KVA_TRY(putf(&ctx->g_out, w->out_norm, d, "out_norm"));
    {
        std::vector<RowSrc> rows;
        add_rows(rows, w->in_proj, d);
        pad_rows(rows);
        KVA_TRY(pack_weight(ctx, dt, n_in, rows, trunk_t, &ctx->w_in, "in_proj"));
    }
    if (!w->blocks) return fail(KVA_ERR_ARG, "blocks is NULL");
    ctx->blk.resize(c.n_blocks);
    for (int b = 0; b < c.n_blocks; ++b) {
        const kva_block_weights& bw = w->blocks[b];
        kva_ctx::Blk& B = ctx->blk[b];
        KVA_TRY(putf(&B.g_attn, bw.attn_norm, d, "attn_norm"));
        KVA_TRY(putf(&B.g_ffn, bw.ffn_norm, d, "ffn_norm"));
        std::vector<RowSrc> rows;
        add_rows(rows, bw.wq, hd);
        add_rows(rows, bw.wk, hd);
        add_rows(rows, bw.wv, hd);
        pad_rows(rows);
        KVA_TRY(pack_weight(ctx, dt, d, rows, trunk_t, &B.wqkv, "wq|wk|wv"));
        rows.clear();
        add_rows(rows, bw.wo, d);
        pad_rows(rows);
        KVA_TRY(pack_weight(ctx, dt, hd, rows, trunk_t, &B.wo, "wo"));
        // gate/up interleaved in groups of 32 rows so one 64-column MFMA pair
        // holds gate and up of the same 32 hidden units
        rows.clear();
        for (int64_t pr = 0; pr < 2 * F; ++pr) {
            const int64_t f = (pr / 64) * 32 + pr % 32;
            rows.push_back({(pr % 64) < 32 ? bw.w_gate : bw.w_up, f});
        }
        pad_rows(rows);
        KVA_TRY(pack_weight(ctx, dt, d, rows, trunk_t, &B.wgu, "w_gate|w_up"));
        rows.clear();
        add_rows(rows, bw.w_down, d);
        pad_rows(rows);
        KVA_TRY(pack_weight(ctx, dt, F, rows, trunk_t, &B.wd, "w_down"));
    }

    // -------- heads, packed column order
    KVA_TRY(pack_heads(ctx, c, w->head_w, w->head_b, d, head_t));

    // -------- scratch
    const int64_t m = round_up(c.max_tokens, kRowPad);
    ctx->m_alloc = m;
    ctx->skinny = c.max_tokens <= kSkinnyTokens;
    ctx->n_split = ctx->skinny ? kSkinnySplits : split_narrow(d, c.max_tokens, ctx->trunk_opd == OPD_F16);
    // The input RMSNorm runs inside the input GEMM (EPI_INPUT), except on the
    // skinny kernel, which reads a normalised fp16 copy
    if (ctx->skinny) HIP_TRY(ctx->alloc(&ctx->u16, (size_t)m * n_in * 2, false));
    else HIP_TRY(ctx->alloc(&ctx->ss_in, (size_t)ctx->n_split * m * 4, false));
    HIP_TRY(ctx->alloc(&ctx->h, (size_t)m * d * 4, false));
    HIP_TRY(ctx->alloc(&ctx->a16, (size_t)m * d * 2, false));
    HIP_TRY(ctx->alloc(&ctx->qk16, (size_t)m * 2 * hd * 2, false));
    HIP_TRY(ctx->alloc(&ctx->vt16, (size_t)hd * m * 2, false));
    HIP_TRY(ctx->alloc(&ctx->o16, (size_t)m * hd * 2, false));
    HIP_TRY(ctx->alloc(&ctx->act16, (size_t)m * F * 2, false));
    HIP_TRY(ctx->alloc(&ctx->z16, (size_t)m * d * 2, false));
    HIP_TRY(ctx->alloc(&ctx->ws, (size_t)ctx->n_split * m * d * 4, false));
    // Scratch rows past n_tokens feed MFMA rows whose results are dropped; zero
    // them once so they always hold finite values.
    if (ctx->u16) HIP_TRY(hipMemset(ctx->u16, 0, (size_t)m * n_in * 2));
    HIP_TRY(hipMemset(ctx->h, 0, (size_t)m * d * 4));
    HIP_TRY(hipMemset(ctx->a16, 0, (size_t)m * d * 2));
    HIP_TRY(hipMemset(ctx->qk16, 0, (size_t)m * 2 * hd * 2));
    HIP_TRY(hipMemset(ctx->vt16, 0, (size_t)hd * m * 2));
    HIP_TRY(hipMemset(ctx->o16, 0, (size_t)m * hd * 2));
    HIP_TRY(hipMemset(ctx->act16, 0, (size_t)m * F * 2));
    HIP_TRY(hipMemset(ctx->z16, 0, (size_t)m * d * 2));
    HIP_TRY(hipDeviceSynchronize());
    return KVA_OK;
}

// Tile for an M x N GEMM with `splits` K-ranges: the one with the fewer
// estimated rounds over the 256 CUs, a 256x256 tile doing the work of four
// 128x128 tiles in about 1/1.3 of their time.  Tile shape never changes a
// result's bits (same K order per output).
// Tile of a four-stage (tiled32) trunk GEMM: 256x256 runs one workgroup per
// CU; 128x128 runs two per CU (64 KB of LDS each), each taking about 1.3 / 4
// of a 256x256 tile's time when alone.  With 16-bit operands (wide_ok), a
// GEMM whose 256x128 tiles still fit one round (the narrow and QKV GEMMs of
// a 1024-token ubatch) takes those instead: half a 256x256 tile's work per CU
// on twice the CUs, 8 waves of 64x64 (measured 8-18% faster per GEMM than
// either alternative there).  Not when 256-row tiles pad more rows than
// 128-row ones.
GemmTile pick_tile_t32(int64_t M, int64_t N, int splits, bool wide_ok) {
    // A call of at most 64 rows: 64-row tiles (no rows computed past the
    // 64th) of 64 columns (128 for SwiGLU), so that a narrow call still
    // spreads its weights over a hundred or more workgroups.
    if (M <= 64 && N % 128 == 0) return TILE_64xN;
    const int64_t t128 = ((M + 127) / 128) * (N / 128) * splits;
    const int64_t t256 = ((M + 255) / 256) * (N / 256) * splits;
    const int64_t t21 = ((M + 255) / 256) * (N / 128) * splits;
    const bool no_extra_pad = M % 256 == 0 || M % 256 > 128;
    if (wide_ok && N % 128 == 0 && no_extra_pad && t21 <= 256) return TILE_256x128;
    const double c256 = (double)((t256 + 255) / 256);
    const double c128 = (double)((t128 + 511) / 512) * 2.0 * 1.3 / 4.0;
    return (N % 256 == 0 && c256 <= c128) ? TILE_256x256 : TILE_128x128;
}


void set_b(GemmArgs& g, const kva_ctx::DevW& w, int64_t K) {
    g.B = w.w16;
    g.Bq = w.q;
    g.Bs = w.sc;
}

// A HIP error left pending on this thread by earlier, unrelated work would be
// returned by the hipGetLastError that follows our launches: clear it first.
inline void clear_stale_error() { (void)hipGetLastError(); }

#define LAUNCH(expr)                                                                      \
    do {                                                                                  \
        hipError_t e_ = (expr);                                                           \
        if (e_ != hipSuccess) return fail(KVA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

// Launch of one stage of the projection, bracketed by an event pair when the
// stage is selected for profiling.
#define STAGE(stage, expr)                                                                \
    do {                                                                                  \
        hipEvent_t a_ = nullptr, b_ = nullptr;                                            \
        if (ctx->prof_mask & (1u << (stage))) {                                           \
            a_ = ctx->take_event();                                                       \
            b_ = ctx->take_event();                                                       \
            if (a_ && b_) HIP_TRY(hipEventRecord(a_, s));                                 \
        }                                                                                 \
        LAUNCH(expr);                                                                     \
        if (a_ && b_) {                                                                   \
            HIP_TRY(hipEventRecord(b_, s));                                               \
            ctx->prof_pending.push_back({(stage), a_, b_});                               \
        }                                                                                 \
    } while (0)

// ------------------------------------------------------------------ static scratch

// Device memory of kva_map_project_noalloc: the tiled 16-bit copy of the
// residual rows that feeds the maps' GEMM (round_up(n_tokens, 256) x n_in
// values), for callers that cannot allocate.  One copy per device, held
// until the process ends; every call on a device shares it.
constexpr uint64_t kStaticScratchBytes = 16ull << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Resolves the device address of `scratch` on `device` (which must be
// current) once; the host-side name of the array is not a device address.
kva_status static_scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return fail(KVA_ERR_UNSUPPORTED, "device index %d", device);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[device]) return KVA_OK;
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(KVA_ERR_HIP, "hipGetSymbolAddress gave NULL for the static scratch");
    g_scratch_ptr[device] = p;
    return KVA_OK;
}

void* static_scratch_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    return g_scratch_ptr[device];
}

// The single-map projection with the residual's tiled copy at `a_buf`
// (round_up(n, 256) x n_in 16-bit values).  `profile`: record the
// kva_profile_* event pairs (kva_map_project_noalloc does not: creating an
// event is a runtime allocation).
kva_status map_project_impl(kva_ctx* ctx, const float* x, int32_t n, float* const* out, uint16_t* a_buf,
                            bool profile, void* stream) {
    const kva_config& c = ctx->cfg;
    if (n < 1 || n > c.max_tokens) return fail(KVA_ERR_SHAPE, "n_tokens %d outside [1, %d]", n, c.max_tokens);
    if ((uintptr_t)x % 16) return fail(KVA_ERR_ARG, "x must be 16-byte aligned (rows are read 16 bytes at a time)");
    HeadOut ho{};
    for (int i = 0; i < c.n_out_heads; ++i) {
        if (!out[i]) return fail(KVA_ERR_ARG, "out[%d] is NULL", i);
        ho.ptr[i] = out[i];
        ho.ld[i] = c.n_in;
    }
    HIP_TRY(hipSetDevice(ctx->device));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t saved_mask = ctx->prof_mask;
    if (!profile) ctx->prof_mask = 0;
    struct Restore {
        kva_ctx* c;
        uint32_t m;
        ~Restore() { c->prof_mask = m; }
    } restore{ctx, saved_mask};
    STAGE(KVA_STAGE_NORM, launch_cast_tiled(x, c.n_in, n, c.n_in, a_buf, !ctx->q8, s));
    GemmArgs g;
    g.A = a_buf; g.lda = c.n_in; set_b(g, ctx->w_heads, c.n_in);
    g.M = n; g.N = (int32_t)ctx->n_pad_heads; g.K = c.n_in;
    g.epi.n_real = (int32_t)ctx->n_pad_heads;
    g.epi.tile_head = ctx->tile_head; g.epi.tile_col0 = ctx->tile_col0;
    g.epi.tail_head = ctx->tail_head; g.epi.tail_col = ctx->tail_col;
    g.epi.tail_start = ctx->tail_start; g.epi.bias = ctx->b_heads;
    g.epi.heads = ho;
    const GemmOperand opd = ctx->q4 ? OPD_Q4 : ctx->q8 ? OPD_Q8 : OPD_BF16;
    STAGE(KVA_STAGE_GEMM_HEADS, launch_gemm_heads(opd, g, ctx->n_cu, 0, s));
    ctx->stats.calls += 1;
    ctx->stats.tokens += (uint64_t)n;
    return KVA_OK;
}

}  // namespace


// ================================================================== C ABI

extern "C" {

kva_status kva_validate_config(const kva_config* cfg) { return validate(cfg); }

kva_status kva_create(const kva_config* cfg, const kva_weights* w, int device, kva_ctx** out) {
    if (!out) return fail(KVA_ERR_ARG, "out is NULL");
    *out = nullptr;
    KVA_TRY(validate(cfg));
    if (!w) return fail(KVA_ERR_ARG, "weights are NULL");
    kva_ctx* ctx = new (std::nothrow) kva_ctx();
    if (!ctx) return fail(KVA_ERR_OOM, "host allocation failed");
    ctx->cfg = *cfg;
    ctx->heads.assign(cfg->out_heads, cfg->out_heads + cfg->n_out_heads);
    ctx->cfg.out_heads = ctx->heads.data();
    kva_status s;
    try {
        s = create_impl(&ctx->cfg, w, device, ctx);
    } catch (const std::bad_alloc&) {
        s = fail(KVA_ERR_OOM, "host allocation failed while repacking weights");
    }
    if (s != KVA_OK) {
        delete ctx;
        return s;
    }
    ctx->stats.weight_bytes = ctx->weight_bytes;
    ctx->stats.scratch_bytes = ctx->scratch_bytes;
    *out = ctx;
    return KVA_OK;
}

namespace {

kva_status check_paged_kv(const kva_paged_kv* cache, const float* k_gain) {
    if (!k_gain || !cache || !cache->k_pool || !cache->v_pool || !cache->page_table)
        return fail(KVA_ERR_ARG, "NULL argument");
    if (cache->n_kv_heads != kKvHeads || cache->head_dim != kKvHeadDim)
        return fail(KVA_ERR_UNSUPPORTED, "only 4 KV heads of 256 dims are supported");
    if (cache->n_rot <= 0 || cache->n_rot > 64 || cache->n_rot % 8)
        return fail(KVA_ERR_SHAPE, "n_rot must be a multiple of 8 in [8, 64]");
    if (cache->page_size <= 0 || cache->n_pages <= 0 || cache->n_logical <= 0)
        return fail(KVA_ERR_SHAPE, "page_size, n_pages and n_logical must be positive");
    if (!(cache->rope_base > 1.0) || !std::isfinite(cache->rope_base))
        return fail(KVA_ERR_ARG, "rope_base must be > 1");
    if ((int64_t)cache->n_logical * cache->page_size > INT32_MAX)
        return fail(KVA_ERR_SHAPE, "n_logical * page_size must stay below 2^31 positions");
    if (cache->kv_type != KVA_KV_BF16 && cache->kv_type != KVA_KV_Q8_0_HADAMARD)
        return fail(KVA_ERR_DTYPE, "unknown kv_type %d", cache->kv_type);
    if (cache->kv_type == KVA_KV_Q8_0_HADAMARD &&
        (((uintptr_t)cache->k_pool | (uintptr_t)cache->v_pool) % 2))
        return fail(KVA_ERR_ARG, "q8_0 pools must be 2-byte aligned");
    return KVA_OK;
}

KvPool make_pool(const kva_paged_kv* cache, const float* k_gain) {
    KvPool p{};
    p.k_pool = cache->k_pool; p.v_pool = cache->v_pool; p.page_table = cache->page_table;
    p.k_gain = k_gain; p.page_size = cache->page_size; p.n_pages = cache->n_pages;
    p.q8 = cache->kv_type == KVA_KV_Q8_0_HADAMARD;
    return p;
}

KvRope make_rope(const kva_paged_kv* cache) {
    KvRope r{};
    r.n_rot = cache->n_rot; r.eps = cache->eps;
    for (int j = 0; j < cache->n_rot / 2; ++j)
        r.inv_freq[j] = std::pow(cache->rope_base, -2.0 * j / (double)cache->n_rot);
    return r;
}

}  // namespace

namespace {

// The projection; with `kv` set, the KV heads' tiles leave through the fused
// KV epilogue instead of as fp32 outputs.
kva_status project(kva_ctx* ctx, const float* x, int32_t n, float* const* head_out, const EpiArgs* kv,
                   void* stream) {
    clear_stale_error();
    if (!ctx || !x || !head_out) return fail(KVA_ERR_ARG, "NULL argument");
    if (ctx->map_only) return fail(KVA_ERR_UNSUPPORTED, "a single-map context has no trunk: use kva_map_project");
    const kva_config& c = ctx->cfg;
    if (n < 1 || n > c.max_tokens)
        return fail(KVA_ERR_SHAPE, "n_tokens %d outside [1, %d]", n, c.max_tokens);
    if ((uintptr_t)x % 16) return fail(KVA_ERR_ARG, "x must be 16-byte aligned (rows are read 16 bytes at a time)");
    HeadOut ho{};
    for (int i = 0; i < c.n_out_heads; ++i) {
        const bool fused = kv && kv->kv_slot[i] >= 0;
        if (!head_out[i] && !fused) return fail(KVA_ERR_ARG, "head_out[%d] is NULL", i);
        ho.ptr[i] = fused ? nullptr : head_out[i];
        ho.ld[i] = c.out_heads[i].out_dim;
    }
    HIP_TRY(hipSetDevice(ctx->device));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t d = c.d_model, F = c.d_ffn, n_in = c.n_in;
    const int64_t hd = (int64_t)c.n_heads * c.head_dim;
    // every GEMM activation operand is written in the tiled32 layout
    const GemmOperand opd = ctx->trunk_opd;
    auto gemm = [&](EpiKind epi, const GemmArgs& g) -> hipError_t {
        if (ctx->skinny) return launch_gemm_skinny(opd, epi, g, s);
        return launch_gemm_t32(opd, pick_tile_t32(g.M, g.N, g.splits, opd == OPD_F16), epi, g, s);
    };
    const int64_t pstride = ctx->m_alloc * d;   // between split-K partial buffers
    // The narrow GEMMs (N = d: input, O, down) write n_split partials to ws;
    // the next norm folds them into h in a fixed order.
    auto narrow = [&](const uint16_t* A, int64_t K, const kva_ctx::DevW& W, int stage) -> kva_status {
        GemmArgs g;
        g.A = A; g.lda = K; set_b(g, W, K);
        g.M = n; g.N = (int32_t)round_up(d, kColPad); g.K = (int32_t)K;
        g.splits = ctx->n_split; g.split_stride = pstride;
        g.epi.out_f32 = ctx->ws; g.epi.ld_f32 = d; g.epi.n_real = (int32_t)d;
        STAGE(stage, gemm(EPI_PARTIAL, g));
        return KVA_OK;
    };
    // ss: the input GEMM's row sums of squares (the first fold applies the
    // input norm's 1/RMS to the summed partials)
    auto fold = [&](bool add, const float* gain, uint16_t* out, bool bf16, const float* ss = nullptr) -> kva_status {
        STAGE(KVA_STAGE_NORM, launch_fold_rmsnorm(ctx->h, d, add, ctx->ws, ctx->n_split, pstride, d, gain, n,
                                                  (int32_t)d, c.eps, out, bf16, s, ss, ctx->m_alloc, (int32_t)n_in));
        return KVA_OK;
    };

    if (ctx->skinny) {
        STAGE(KVA_STAGE_NORM,
              launch_rmsnorm_cast(x, n_in, ctx->g_in, n, (int32_t)n_in, c.eps, ctx->u16, false, s));
        KVA_TRY(narrow(ctx->u16, n_in, ctx->w_in, KVA_STAGE_GEMM_IN));
    } else {
        // RMSNorm + input Linear in one GEMM: A = fp16(x * g_in), unnormalised
        // partials, and each row's sum of squares for the fold
        GemmArgs g;
        g.A = reinterpret_cast<const uint16_t*>(x); g.lda = n_in; set_b(g, ctx->w_in, n_in);
        g.M = n; g.N = (int32_t)round_up(d, kColPad); g.K = (int32_t)n_in;
        g.splits = ctx->n_split; g.split_stride = pstride;
        g.epi.out_f32 = ctx->ws; g.epi.ld_f32 = d; g.epi.n_real = (int32_t)d;
        g.epi.a_gain = ctx->g_in; g.epi.ss = ctx->ss_in; g.epi.ss_stride = ctx->m_alloc;
        // The input kernel keeps three slabs of both operands in registers
        // (a 256x256 tile's accumulators leave no room for them: the compiler
        // then waits for every load in flight), and its time follows the
        // bytes it copies per slab, of which the fp32 rows are most: with
        // 16-bit weights the 256-row tiles take 128x256 ones instead (32 KB a
        // slab for the work of a 256x128 tile's 40 KB); code-plane contexts
        // (at most 256 tokens per call) take 128x128 for a 256x256 choice.
        // Same bits: one K order and one sum-of-squares order for every tile.
        GemmTile t = pick_tile_t32(g.M, g.N, g.splits, opd == OPD_F16);
        if (opd == OPD_F16 && (t == TILE_256x256 || t == TILE_256x128) && g.N % 256 == 0) t = TILE_128x256;
        if (opd != OPD_F16 && t == TILE_256x256) t = TILE_128x128;
        STAGE(KVA_STAGE_GEMM_IN, launch_gemm_t32(opd, t, EPI_INPUT, g, s));
    }
    for (int b = 0; b < c.n_blocks; ++b) {
        const kva_ctx::Blk& B = ctx->blk[b];
        // h = (b == 0 ? 0 : h) + input/down partials; a = attn_norm(h)
        KVA_TRY(fold(b > 0, B.g_attn, ctx->a16, false, (b == 0 && !ctx->skinny) ? ctx->ss_in : nullptr));
        {
            GemmArgs g;
            g.A = ctx->a16; g.lda = d; set_b(g, B.wqkv, d);
            g.M = n; g.N = (int32_t)round_up(3 * hd, kColPad); g.K = (int32_t)d;
            g.epi.out16 = ctx->qk16; g.epi.ld16 = 2 * hd;
            g.epi.vt = ctx->vt16; g.epi.ld_vt = ctx->m_alloc; g.epi.n_split = (int32_t)(2 * hd);
            g.epi.n_real = (int32_t)(3 * hd);
            STAGE(KVA_STAGE_GEMM_QKV, gemm(EPI_QKV, g));
        }
        STAGE(KVA_STAGE_ATTN, launch_attention(ctx->qk16, 2 * hd, (int32_t)hd, ctx->vt16, ctx->m_alloc, ctx->o16, hd, n,
                                               c.n_heads, c.attn_block, s));
        KVA_TRY(narrow(ctx->o16, hd, B.wo, KVA_STAGE_GEMM_O));
        KVA_TRY(fold(true, B.g_ffn, ctx->a16, false));           // h += O partials; a = ffn_norm(h)
        {
            GemmArgs g;
            g.A = ctx->a16; g.lda = d; set_b(g, B.wgu, d);
            g.M = n; g.N = (int32_t)round_up(2 * F, kColPad); g.K = (int32_t)d;
            g.epi.out16 = ctx->act16; g.epi.ld16 = F; g.epi.n_real = (int32_t)(2 * F);
            STAGE(KVA_STAGE_GEMM_GATEUP, gemm(EPI_SWIGLU, g));
        }
        KVA_TRY(narrow(ctx->act16, F, B.wd, KVA_STAGE_GEMM_DOWN));
    }
    // h += down partials; z = out_norm(h), tiled: bf16, or fp16 for q8_0
    KVA_TRY(fold(true, ctx->g_out, ctx->z16, !ctx->q8));
    {
        GemmArgs g;
        g.A = ctx->z16; g.lda = d; set_b(g, ctx->w_heads, d);
        g.M = n; g.N = (int32_t)ctx->n_pad_heads; g.K = (int32_t)d;
        g.epi.n_real = (int32_t)ctx->n_pad_heads;
        g.epi.tile_head = ctx->tile_head; g.epi.tile_col0 = ctx->tile_col0;
        g.epi.tail_head = ctx->tail_head; g.epi.tail_col = ctx->tail_col;
        g.epi.tail_start = ctx->tail_start; g.epi.bias = ctx->b_heads;
        g.epi.heads = ho;
        if (kv) {
            g.epi.kv_n = kv->kv_n;
            g.epi.kv_pos0 = kv->kv_pos0;
            std::memcpy(g.epi.kv_slot, kv->kv_slot, sizeof(g.epi.kv_slot));
            std::memcpy(g.epi.kv_pool, kv->kv_pool, sizeof(g.epi.kv_pool));
            g.epi.kv_rope = kv->kv_rope;
        }
        STAGE(KVA_STAGE_GEMM_HEADS, launch_gemm_heads(ctx->head_opd, g, ctx->n_cu,
                                                      kv ? ctx->kv_tiles : 0, s));
    }
    ctx->stats.calls += 1;
    ctx->stats.tokens += (uint64_t)n;
    ctx->stats.blocks += (uint64_t)((n + c.attn_block - 1) / c.attn_block);
    return KVA_OK;
}

}  // namespace

kva_status kva_project_ubatch(kva_ctx* ctx, const float* x, int32_t n, float* const* head_out,
                              void* stream) {
    return project(ctx, x, n, head_out, nullptr, stream);
}

kva_status kva_project_ubatch_kv(kva_ctx* ctx, const float* x, int32_t n, float* const* head_out,
                                 int64_t pos0, const kva_attn_dest* attn, int32_t n_attn, void* stream) {
    if (!ctx || !attn) return fail(KVA_ERR_ARG, "NULL argument");
    if (n_attn != (int32_t)ctx->kv_heads.size())
        return fail(KVA_ERR_SHAPE, "n_attn %d, but the projector has %d attention heads of k|v 4 x 256",
                    n_attn, (int)ctx->kv_heads.size());
    if (n_attn > kMaxAttnHeads) return fail(KVA_ERR_UNSUPPORTED, "more than %d attention heads", kMaxAttnHeads);
    if (pos0 < 0) return fail(KVA_ERR_SHAPE, "negative pos0");
    EpiArgs kv{};
    kv.kv_n = n_attn;
    kv.kv_pos0 = pos0;
    std::memset(kv.kv_slot, -1, sizeof(kv.kv_slot));
    for (int a = 0; a < n_attn; ++a) {
        const kva_paged_kv* cache = &attn[a].cache;
        KVA_TRY(check_paged_kv(cache, attn[a].k_gain));
        if (pos0 + n > (int64_t)cache->n_logical * cache->page_size)
            return fail(KVA_ERR_SHAPE, "attention head %d: positions past the page table", a);
        if (cache->n_rot != attn[0].cache.n_rot || cache->rope_base != attn[0].cache.rope_base ||
            cache->eps != attn[0].cache.eps)
            return fail(KVA_ERR_UNSUPPORTED, "attention heads must share n_rot, rope_base and eps");
        kv.kv_slot[ctx->kv_heads[a]] = (int8_t)a;
        kv.kv_pool[a] = make_pool(cache, attn[a].k_gain);
    }
    if (n_attn > 0) kv.kv_rope = make_rope(&attn[0].cache);
    return project(ctx, x, n, head_out, n_attn > 0 ? &kv : nullptr, stream);
}

kva_status kva_map_create(int32_t n_in, int32_t n_maps, int32_t weight_dtype, const void* const* w,
                          const float* const* b, int32_t max_tokens, int device, kva_ctx** out) {
    if (!out) return fail(KVA_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (n_in < 32 || n_in % 32) return fail(KVA_ERR_SHAPE, "n_in must be a positive multiple of 32");
    if (n_maps < 1 || n_maps > kMaxHeads) return fail(KVA_ERR_SHAPE, "n_maps outside [1, %d]", kMaxHeads);
    if (max_tokens < 1) return fail(KVA_ERR_SHAPE, "max_tokens must be positive");
    if (weight_dtype != KVA_DTYPE_F32 && weight_dtype != KVA_DTYPE_BF16 && weight_dtype != KVA_DTYPE_Q8_0 &&
        weight_dtype != KVA_DTYPE_Q4_0)
        return fail(KVA_ERR_DTYPE, "unknown weight_dtype %d", weight_dtype);
    if (!w) return fail(KVA_ERR_ARG, "weights are NULL");
    kva_ctx* ctx = new (std::nothrow) kva_ctx();
    if (!ctx) return fail(KVA_ERR_OOM, "host allocation failed");
    ctx->map_only = true;
    kva_config& c = ctx->cfg;
    c.n_in = n_in;
    c.d_model = n_in;
    c.max_tokens = max_tokens;
    c.weight_dtype = weight_dtype;
    c.has_head_bias = b ? 1 : 0;
    c.n_out_heads = n_maps;
    for (int i = 0; i < n_maps; ++i) ctx->heads.push_back(kva_head_desc{KVA_HEAD_DRAFT, i, n_in});
    c.out_heads = ctx->heads.data();
    kva_status st = KVA_OK;
    try {
        st = [&]() -> kva_status {
            HIP_TRY(hipSetDevice(device));
            ctx->device = device;
            HIP_TRY(hipDeviceGetAttribute(&ctx->n_cu, hipDeviceAttributeMultiprocessorCount, device));
            KVA_TRY(static_scratch_setup(device));
            ctx->q4 = weight_dtype == KVA_DTYPE_Q4_0;
            ctx->q8 = weight_dtype == KVA_DTYPE_Q8_0 || ctx->q4;
            const PackTarget head_t = ctx->q4 ? PACK_Q4 : ctx->q8 ? PACK_Q8 : PACK_BF16_T32;
            KVA_TRY(pack_heads(ctx, c, w, b, n_in, head_t));
            const int64_t m = round_up(max_tokens, kRowPad);
            ctx->m_alloc = m;
            HIP_TRY(ctx->alloc(&ctx->z16, (size_t)m * n_in * 2, false));
            HIP_TRY(hipMemset(ctx->z16, 0, (size_t)m * n_in * 2));
            HIP_TRY(hipDeviceSynchronize());
            return KVA_OK;
        }();
    } catch (const std::bad_alloc&) {
        st = fail(KVA_ERR_OOM, "host allocation failed while repacking weights");
    }
    if (st != KVA_OK) {
        delete ctx;
        return st;
    }
    ctx->stats.weight_bytes = ctx->weight_bytes;
    ctx->stats.scratch_bytes = ctx->scratch_bytes;
    *out = ctx;
    return KVA_OK;
}

kva_status kva_map_project(kva_ctx* ctx, const float* x, int32_t n, float* const* out, void* stream) {
    clear_stale_error();
    if (!ctx || !x || !out) return fail(KVA_ERR_ARG, "NULL argument");
    if (!ctx->map_only) return fail(KVA_ERR_UNSUPPORTED, "not a single-map context (see kva_map_create)");
    return map_project_impl(ctx, x, n, out, ctx->z16, true, stream);
}

kva_status kva_map_project_noalloc(kva_ctx* ctx, const float* x, int32_t n, float* const* out, void* stream) {
    clear_stale_error();
    if (!ctx || !x || !out) return fail(KVA_ERR_ARG, "NULL argument");
    if (!ctx->map_only) return fail(KVA_ERR_UNSUPPORTED, "not a single-map context (see kva_map_create)");
    if (n < 1 || n > ctx->cfg.max_tokens)
        return fail(KVA_ERR_SHAPE, "n_tokens %d outside [1, %d]", n, ctx->cfg.max_tokens);
    const uint64_t need = (uint64_t)round_up(n, kRowPad) * (uint64_t)ctx->cfg.n_in * 2u;
    if (need > kStaticScratchBytes)
        return fail(KVA_ERR_SHAPE, "n_tokens %d needs %llu bytes of the static scratch, which holds %llu", n,
                    (unsigned long long)need, (unsigned long long)kStaticScratchBytes);
    void* buf = static_scratch_ptr(ctx->device);
    if (!buf) return fail(KVA_ERR_HIP, "the static scratch of device %d has no address (see kva_map_create)",
                          ctx->device);
    return map_project_impl(ctx, x, n, out, static_cast<uint16_t*>(buf), false, stream);
}

kva_status kva_destroy(kva_ctx* ctx) {
    if (!ctx) return KVA_OK;
    kva_status s = KVA_OK;
    if (hipSetDevice(ctx->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
        s = fail(KVA_ERR_HIP, "device synchronisation failed in kva_destroy");
    delete ctx;
    return s;
}

kva_status kva_attn_kv_write(const float* kv, int64_t ld_kv, int32_t n, int64_t pos0,
                             const float* k_gain, const kva_paged_kv* cache, void* stream) {
    clear_stale_error();
    if (!kv) return fail(KVA_ERR_ARG, "NULL argument");
    KVA_TRY(check_paged_kv(cache, k_gain));
    if (n < 0 || pos0 < 0) return fail(KVA_ERR_SHAPE, "negative n_tokens or pos0");
    if (ld_kv < 2LL * cache->n_kv_heads * cache->head_dim || ld_kv % 4)
        return fail(KVA_ERR_SHAPE, "ld_kv must be >= 2*n_kv_heads*head_dim and a multiple of 4");
    if (pos0 + n > (int64_t)cache->n_logical * cache->page_size)
        return fail(KVA_ERR_SHAPE, "positions past the page table");
    if (n == 0) return KVA_OK;
    KvWriteArgs a{};
    a.kv = kv; a.ld_kv = ld_kv; a.n_tokens = n; a.pos0 = pos0;
    a.pool = make_pool(cache, k_gain);
    a.rope = make_rope(cache);
    LAUNCH(launch_kv_write(a, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_deltanet_update(const kva_deltanet_layer* layers, int32_t n_layers, int32_t n_tokens,
                               int32_t n_k_heads, int32_t n_v_heads, int32_t head_dim, void* stream) {
    clear_stale_error();
    if (n_layers < 0 || n_tokens < 0) return fail(KVA_ERR_SHAPE, "negative n_layers or n_tokens");
    if (n_layers == 0 || n_tokens == 0) return KVA_OK;
    if (!layers) return fail(KVA_ERR_ARG, "NULL layers");
    if (head_dim != kDnHeadDim) return fail(KVA_ERR_UNSUPPORTED, "head_dim must be %d", kDnHeadDim);
    if (n_k_heads <= 0 || n_v_heads <= 0 || n_v_heads % n_k_heads)
        return fail(KVA_ERR_SHAPE, "n_v_heads must be a positive multiple of n_k_heads");
    if (n_v_heads / n_k_heads > 3)
        return fail(KVA_ERR_UNSUPPORTED, "at most 3 value heads per key head are supported");
    const int64_t qkv = (int64_t)(2 * n_k_heads + n_v_heads) * head_dim;
    for (int l = 0; l < n_layers; ++l) {
        const kva_deltanet_layer& L = layers[l];
        if (!L.mixer_in || !L.conv_w || !L.a_log || !L.dt_bias || !L.conv_state || !L.state)
            return fail(KVA_ERR_ARG, "layer %d: NULL pointer", l);
        if (L.ld_in < qkv + 2 * n_v_heads) return fail(KVA_ERR_SHAPE, "layer %d: ld_in too small", l);
        if ((uintptr_t)L.conv_w % 16 || (uintptr_t)L.mixer_in % 4 || (uintptr_t)L.state % 4 ||
            (uintptr_t)L.conv_state % 4)
            return fail(KVA_ERR_ARG, "layer %d: misaligned pointer (conv_w needs 16 bytes)", l);
    }
    for (int l0 = 0; l0 < n_layers; l0 += kMaxDnLayers) {
        DnArgs a{};
        a.n_tokens = n_tokens;
        a.n_layers = n_layers - l0 < kMaxDnLayers ? n_layers - l0 : kMaxDnLayers;
        a.n_k = n_k_heads;
        a.n_v = n_v_heads;
        for (int l = 0; l < a.n_layers; ++l) {
            const kva_deltanet_layer& L = layers[l0 + l];
            a.layer[l] = DnLayer{L.mixer_in, L.ld_in, L.conv_w, L.a_log, L.dt_bias, L.conv_state, L.state};
        }
        LAUNCH(launch_deltanet_update(a, static_cast<hipStream_t>(stream)));
    }
    return KVA_OK;
}

kva_status kva_debug_dequant_q8_0(const void* blocks, int64_t n_blocks, float* out, void* stream) {
    clear_stale_error();
    if (!blocks || !out) return fail(KVA_ERR_ARG, "NULL argument");
    if (n_blocks < 0) return fail(KVA_ERR_SHAPE, "negative n_blocks");
    LAUNCH(launch_dequant_q8_0(blocks, n_blocks, out, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_dequant_q4_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, void* stream) {
    clear_stale_error();
    if (!blocks || !out) return fail(KVA_ERR_ARG, "NULL argument");
    if (n_blocks < 0) return fail(KVA_ERR_SHAPE, "negative n_blocks");
    LAUNCH(launch_dequant_q4_0_f16(blocks, n_blocks, out, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_dequant_q8_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, void* stream) {
    clear_stale_error();
    if (!blocks || !out) return fail(KVA_ERR_ARG, "NULL argument");
    if (n_blocks < 0) return fail(KVA_ERR_SHAPE, "negative n_blocks");
    LAUNCH(launch_dequant_q8_0_f16(blocks, n_blocks, out, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_check_q8_scale(unsigned long long* counts, void* stream) {
    clear_stale_error();
    if (!counts) return fail(KVA_ERR_ARG, "NULL argument");
    LAUNCH(launch_check_q8_scale(counts, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_mfma_loop(int32_t n_iter, int32_t n_workgroups, float* sink, void* stream) {
    clear_stale_error();
    if (!sink) return fail(KVA_ERR_ARG, "NULL argument");
    if (n_iter <= 0 || n_workgroups <= 0) return fail(KVA_ERR_SHAPE, "n_iter and n_workgroups must be positive");
    LAUNCH(launch_mfma_loop(n_iter, n_workgroups, sink, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_copy_z(kva_ctx* ctx, uint16_t* dst, int32_t n, void* stream) {
    clear_stale_error();
    if (!ctx || !dst) return fail(KVA_ERR_ARG, "NULL argument");
    if (n < 1 || n > ctx->cfg.max_tokens) return fail(KVA_ERR_SHAPE, "bad n_tokens");
    LAUNCH(launch_untile32(ctx->z16, dst, n, ctx->cfg.d_model, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_poison_scratch(kva_ctx* ctx, void* stream) {
    clear_stale_error();
    if (!ctx) return fail(KVA_ERR_ARG, "NULL argument");
    HIP_TRY(hipSetDevice(ctx->device));
    for (const auto& r : ctx->scratch_regions)
        HIP_TRY(hipMemsetAsync(r.first, 0xFF, r.second, static_cast<hipStream_t>(stream)));
    return KVA_OK;
}

kva_status kva_debug_head_plan(const kva_config* cfg, int32_t* n_cols, int32_t* col_head,
                               int32_t* col_index, int64_t capacity) {
    KVA_TRY(validate(cfg));
    if (!n_cols) return fail(KVA_ERR_ARG, "n_cols is NULL");
    HeadPlan p = plan_heads(*cfg);
    *n_cols = (int32_t)p.n_pad;
    if (!col_head && !col_index) return KVA_OK;
    if (capacity < p.n_pad) return fail(KVA_ERR_SHAPE, "capacity %lld < %lld", (long long)capacity, (long long)p.n_pad);
    for (int64_t i = 0; i < p.n_pad; ++i) {
        if (col_head) col_head[i] = p.col_head[i];
        if (col_index) col_index[i] = p.col_head[i] < 0 ? -1 : p.col_index[i];
    }
    return KVA_OK;
}

kva_status kva_debug_pack_weight(const void* src, int32_t src_dtype, int32_t rows, int32_t K, int32_t target,
                                 void* out, int64_t out_bytes, uint16_t* scales, int64_t n_scales) {
    if (!src || !out) return fail(KVA_ERR_ARG, "NULL argument");
    if (rows <= 0 || K <= 0) return fail(KVA_ERR_SHAPE, "rows and K must be positive");
    if (target < PACK_F16_T32 || target > PACK_Q4) return fail(KVA_ERR_ARG, "unknown target %d", target);
    std::vector<RowSrc> rv;
    for (int32_t r = 0; r < rows; ++r) rv.push_back({src, r});
    while (rv.size() % kColPad) rv.push_back({nullptr, -1});
    HostPacked hp;
    try {
        KVA_TRY(pack_host(src_dtype, K, rv, (PackTarget)target, &hp, "debug"));
    } catch (const std::bad_alloc&) {
        return fail(KVA_ERR_OOM, "host allocation failed");
    }
    const bool quant = target == PACK_Q8 || target == PACK_Q4;
    const size_t bytes = quant ? hp.q.size() : hp.w16.size() * 2;
    if ((uint64_t)out_bytes < bytes) return fail(KVA_ERR_SHAPE, "out needs %zu bytes", bytes);
    std::memcpy(out, quant ? (const void*)hp.q.data() : (const void*)hp.w16.data(), bytes);
    if (quant) {
        if (!scales || n_scales < (int64_t)hp.sc.size())
            return fail(KVA_ERR_SHAPE, "scales needs %zu entries", hp.sc.size());
        std::memcpy(scales, hp.sc.data(), hp.sc.size() * 2);
    }
    return KVA_OK;
}

kva_status kva_debug_host_to_f16(const void* src, int32_t src_dtype, int64_t n, uint16_t* dst) {
    if (!src || !dst) return fail(KVA_ERR_ARG, "NULL argument");
    if (src_dtype != KVA_DTYPE_F32 && src_dtype != KVA_DTYPE_BF16) return fail(KVA_ERR_DTYPE, "bad dtype");
    bool ovf = false;
    for (int64_t i = 0; i < n; ++i) dst[i] = f32_to_f16(load_f32(src, src_dtype, i), &ovf);
    return ovf ? fail(KVA_ERR_RANGE, "value outside the fp16 range") : KVA_OK;
}

kva_status kva_profile_enable(kva_ctx* ctx, uint32_t stage_mask) {
    if (!ctx) return fail(KVA_ERR_ARG, "ctx is NULL");
    ctx->prof_mask = stage_mask & ((1u << KVA_N_STAGES) - 1u);
    return KVA_OK;
}

kva_status kva_profile_read(kva_ctx* ctx, kva_stage_time* out) {
    if (!ctx || !out) return fail(KVA_ERR_ARG, "NULL argument");
    HIP_TRY(hipSetDevice(ctx->device));
    for (kva_ctx::Rec& r : ctx->prof_pending) {
        HIP_TRY(hipEventSynchronize(r.b));
        float ms = 0.0f;
        HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
        ctx->prof_acc[r.stage].launches += 1;
        ctx->prof_acc[r.stage].total_ms += ms;
        ctx->prof_free.push_back(r.a);
        ctx->prof_free.push_back(r.b);
    }
    ctx->prof_pending.clear();
    for (int i = 0; i < KVA_N_STAGES; ++i) {
        out[i] = ctx->prof_acc[i];
        ctx->prof_acc[i] = kva_stage_time{};
    }
    return KVA_OK;
}

kva_status kva_get_stats(const kva_ctx* ctx, kva_stats* out) {
    if (!ctx || !out) return fail(KVA_ERR_ARG, "NULL argument");
    *out = ctx->stats;
    return KVA_OK;
}

const char* kva_status_str(kva_status s) {
    switch (s) {
        case KVA_OK: return "KVA_OK";
        case KVA_ERR_ARG: return "KVA_ERR_ARG";
        case KVA_ERR_SHAPE: return "KVA_ERR_SHAPE";
        case KVA_ERR_DTYPE: return "KVA_ERR_DTYPE";
        case KVA_ERR_OOM: return "KVA_ERR_OOM";
        case KVA_ERR_RANGE: return "KVA_ERR_RANGE";
        case KVA_ERR_UNSUPPORTED: return "KVA_ERR_UNSUPPORTED";
        case KVA_ERR_HIP: return "KVA_ERR_HIP";
    }
    return "KVA_ERR_UNKNOWN";
}

const char* kva_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
