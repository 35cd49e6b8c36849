// Internal declarations shared by the runtime (kva_runtime.hip) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kva {

constexpr int kMaxHeads = 64;
// Column tile of the head GEMM.  Head outputs are packed so that every tile
// belongs to one head, except the "tail" tiles that gather the out_dim % 256
// remainders of all heads (e.g. the 24 DeltaNet a|b pairs, 24 * 96 columns).
constexpr int kHeadTileN = 256;
// Activation scratch is allocated with rows rounded up to this, so GEMM A
// tiles never need a row clamp (rows >= n_tokens are computed and dropped).
constexpr int kRowPad = 256;
// Weight rows are padded with zeros to a multiple of this.
constexpr int kColPad = 256;
// 16-bit GEMM operands [rows][K] (weights, and the activations that feed a
// GEMM with 16-bit weights) are stored tiled: for each group of
// kWeightTileRows rows and each 32-wide K slab, one contiguous block of
// kWeightTileRows x 32 values, row after row (64-byte rows); within a row the
// 16-byte chunk c (K-values 8c..8c+7) sits at chunk c ^ tiled32_swizzle(r).
// That is exactly the LDS layout of a gemm_t32 slab, so every operand DMA
// instruction reads one contiguous kilobyte.
constexpr int kWeightTileRows = 256;
// Attention's softmax works in base 2 on q.k / sqrt(128): the QKV GEMM
// writes Q already multiplied by log2(e) / sqrt(128) (before its fp16
// rounding), so the attention kernel exponentiates its scores directly.
constexpr float kAttnQScale = 0.12751743082459868f;
// The chunk rotation of row r: bits 2 and 3 of the row.  A wave's MFMA
// fragment read (32 rows, 16 bytes each, two chunks per row across the two
// lane halves) then falls on distinct LDS banks; the earlier rotation
// ((r >> 1) ^ (r >> 3)) & 3 left every such read 2-way conflicted on gfx950
// (measured with the SQ_LDS_BANK_CONFLICT counter).
__host__ __device__ inline int tiled32_swizzle(int64_t r) { return (int)((r >> 2) & 3); }
__host__ __device__ inline int64_t tiled32_index(int64_t row, int64_t k, int64_t K) {
    const int64_t nb = row / kWeightTileRows, r = row % kWeightTileRows, kt = k / 32;
    const int64_t c = (k % 32) / 8, e = k % 8;
    const int64_t sw = tiled32_swizzle(r);
    return ((nb * (K / 32) + kt) * kWeightTileRows + r) * 32 + ((c ^ sw) * 8) + e;
}
// q8_0 weights [rows][K] use the same grouping: for each 256-row group and
// each 32-wide K slab (exactly one q8_0 block per row), the int8 codes of the
// 256 rows form one contiguous 8 KB block of 32-byte rows, the 8-byte chunk c
// of row r (K-values 8c..8c+7, in q8_chunk_pack order) at chunk
// c ^ ((r >> 2) & 3); the fp16 scales of the same rows form one contiguous
// 512-byte block.  Returns the byte offset of the chunk holding K-value k.
__host__ __device__ inline int64_t q8_code_chunk(int64_t row, int64_t k, int64_t K) {
    const int64_t nb = row / kWeightTileRows, r = row % kWeightTileRows, kt = k / 32;
    const int64_t c = (k % 32) / 8;
    return ((nb * (K / 32) + kt) * kWeightTileRows + r) * 32 + ((c ^ ((r >> 2) & 3)) * 8);
}
// The 8-byte chunk of 8 int8 codes (q[e] = code of K-value 8c + e), each
// stored as the unsigned byte q + 128 (q ^ 0x80): each 32-bit half holds
// codes 4j, 4j + 2, 4j + 1, 4j + 3 in its bytes 0..3, so that one byte
// permute puts a pair of consecutive codes into the two 16-bit halves.
__host__ __device__ inline void q8_chunk_pack(const int8_t q[8], uint32_t* c0, uint32_t* c1) {
    uint32_t w[2];
    for (int j = 0; j < 2; ++j)
        w[j] = (uint32_t)(uint8_t)(q[4 * j] ^ 0x80) | ((uint32_t)(uint8_t)(q[4 * j + 2] ^ 0x80) << 8) |
               ((uint32_t)(uint8_t)(q[4 * j + 1] ^ 0x80) << 16) | ((uint32_t)(uint8_t)(q[4 * j + 3] ^ 0x80) << 24);
    *c0 = w[0];
    *c1 = w[1];
}
__host__ __device__ inline int64_t q8_scale_index(int64_t row, int64_t kblock, int64_t K) {
    return ((row / kWeightTileRows) * (K / 32) + kblock) * kWeightTileRows + row % kWeightTileRows;
}
// q4_0 weights: per 256-row group and 32-wide slab, the codes of the 256
// rows form one contiguous 4 KB block of 16-byte rows; the 32-bit chunk c of
// row r (K-values 8c..8c+7) sits at chunk c ^ ((r >> 3) & 3), with K-value
// 8c + 2h in bits 4h..4h+3 and 8c + 2h + 1 in bits 16+4h..16+4h+3 (h < 4),
// so that one mask puts a pair of codes into the two 16-bit halves.  The
// scales use q8_scale_index.  Returns the byte offset of the chunk holding
// K-value k.
__host__ __device__ inline int64_t q4_code_chunk(int64_t row, int64_t k, int64_t K) {
    const int64_t nb = row / kWeightTileRows, r = row % kWeightTileRows, kt = k / 32;
    const int64_t c = (k % 32) / 8;
    return ((nb * (K / 32) + kt) * kWeightTileRows + r) * 16 + ((c ^ ((r >> 3) & 3)) * 4);
}
// The 32-bit chunk of 8 codes (n[e] = code of K-value 8c + e) in that order.
__host__ __device__ inline uint32_t q4_chunk_pack(const uint8_t n[8]) {
    uint32_t w = 0;
    for (int h = 0; h < 4; ++h)
        w |= ((uint32_t)(n[2 * h] & 0xF) << (4 * h)) | ((uint32_t)(n[2 * h + 1] & 0xF) << (16 + 4 * h));
    return w;
}

// Attention-layer KV cache (4 KV heads of 256 dims per token).
constexpr int kKvHeads = 4;
constexpr int kKvHeadDim = 256;
constexpr int kMaxAttnHeads = 16;

// One attention layer's paged pools, its page table and its k_norm gain
// [kKvHeadDim].  Pools are [n_pages][page_size][kKvHeads][row], a row being
// kKvHeadDim bf16 values, or (q8 != 0) the Hadamard-rotated values as
// kKvHeadDim / 32 q8_0 blocks of 34 bytes.
constexpr int kKvQ8RowBytes = kKvHeadDim / 32 * 34;
struct KvPool {
    void* k_pool;
    void* v_pool;
    const int32_t* page_table;
    const float* k_gain;
    int32_t page_size;
    int32_t n_pages;
    int32_t q8;
};

struct KvRope {
    int32_t n_rot;          // rotary dims at the start of each KV head (multiple of 8, <= 64)
    float eps;              // k_norm epsilon
    double inv_freq[32];    // rope_base^(-2j/n_rot), computed on the host in double
};

struct HeadOut {
    float* ptr[kMaxHeads];
    int32_t ld[kMaxHeads];
};

enum EpiKind : int {
    EPI_QKV = 2,        // n < n_split: out16[m][n] = fp16(acc); else vt[n - n_split][m] = fp16(acc)
    EPI_SWIGLU = 3,     // gate/up interleaved per 32 columns: out16[tiled32_index(m, f, ld16)] = fp16(silu(g) * u)
    EPI_HEADS = 4,      // bias add, scatter to per-head fp32 outputs
    EPI_PARTIAL = 5,    // split-K partial: out_f32[split * split_stride + m * ld_f32 + n] = acc
    // The input Linear with its RMSNorm folded in: A is read as fp32 rows
    // (A = x, lda in floats, 16-byte aligned) and each operand value is
    // formed in the kernel as fp16(x[m][k] * a_gain[k]); the output is the
    // split-K partial of EPI_PARTIAL (unnormalised), and the workgroups of
    // the first N-tile also write each row's sum of squares of x over the
    // split's K range to ss[split * ss_stride + m].  The row's 1/RMS is then
    // applied to the summed partials by the fold (launch_fold_rmsnorm).
    EPI_INPUT = 6
};

struct EpiArgs {
    float* out_f32 = nullptr;
    int64_t ld_f32 = 0;
    uint16_t* out16 = nullptr;
    int64_t ld16 = 0;
    uint16_t* vt = nullptr;
    int64_t ld_vt = 0;
    int32_t n_split = 0;
    int32_t n_real = 0;                 // real (unpadded) columns of the product
    const int32_t* tile_head = nullptr; // per 256-column tile: head, or -1 for a tail tile
    const int32_t* tile_col0 = nullptr; // per tile: first destination column in that head
    const int32_t* tail_head = nullptr; // per tail column: head, or -1 for padding
    const int32_t* tail_col = nullptr;  // per tail column: destination column
    int32_t tail_start = 0;             // first packed column of the tail segment
    const float* bias = nullptr;        // [n_pad] packed bias, or nullptr
    HeadOut heads;
    // Fused attention-layer epilogue (EPI_HEADS): a head with kv_slot[h] >= 0
    // is not written as fp32; its packed tiles (256 columns = one KV head of
    // k, tiles 0..3, or of v, tiles 4..7) go through k_norm + RoPE (k) and
    // bf16 rounding into kv_pool[kv_slot[h]], token m at position kv_pos0 + m.
    int32_t kv_n = 0;                   // 0: no fused epilogue
    int64_t kv_pos0 = 0;
    int8_t kv_slot[kMaxHeads];
    KvPool kv_pool[kMaxAttnHeads];
    KvRope kv_rope;
    // EPI_INPUT: the input norm's gain [K] and the per-split row sums of squares
    const float* a_gain = nullptr;
    float* ss = nullptr;
    int64_t ss_stride = 0;
};

// C[M][N] = A[M][K] * B[N][K]^T with 16-bit activations (tiled32 layout)
// and fp32 accumulation.  16-bit weights: B (tiled32 layout).  q8_0 weights:
// int8 codes Bq (q8_code_chunk layout) and one fp16 scale per 32 codes, Bs
// (q8_scale_index layout); the weight is d * q (see q8_0_value), rounded
// once to fp16 for the MFMA.  q4_0 weights: codes in Bq (q4_code_byte
// layout), scales in Bs as for q8_0.
struct GemmArgs {
    const uint16_t* A = nullptr;
    int64_t lda = 0;
    const uint16_t* B = nullptr;
    const int8_t* Bq = nullptr;
    const uint16_t* Bs = nullptr;
    int32_t M = 0;       // rows of A that are real (stores are masked to M)
    int32_t N = 0;       // columns, a multiple of the tile width (weights are padded)
    int32_t K = 0;       // multiple of 32
    // Split-K: the K slabs are cut into `splits` consecutive ranges, one per
    // workgroup; each range's partial product goes to its own buffer
    // (EPI_PARTIAL).  The split count must depend only on (N, K), never on M,
    // so a row's result never depends on how many rows a call holds.
    int32_t splits = 1;
    int64_t split_stride = 0;
    EpiArgs epi;
};

// Operand type: both operands fp16, both bf16, or fp16 activations with
// q8_0 / q4_0 weights (fp16 MFMA on the weights rounded once to fp16).
enum GemmOperand : int { OPD_F16 = 0, OPD_BF16 = 1, OPD_Q8 = 2, OPD_Q4 = 3 };

// One q8_0 weight: the fp16 block scale (bit pattern d_bits) times the int8
// code, exactly (an 11-bit significand times an 8-bit integer fits fp32's 24
// bits; fp16 subnormal scales convert exactly to fp32).
__device__ __forceinline__ float q8_0_value(uint16_t d_bits, int q) {
    return (float)__builtin_bit_cast(_Float16, d_bits) * (float)q;
}

// Eight q4_0 weights as the fp16 values the MFMA consumes: a chunk of 8
// codes n (q4_chunk_pack order) times the fp16 scale d_bits as d * (n - 8),
// rounded once to nearest-even fp16.  Each code pair goes into the mantissas
// of two fp16 values 1024 + n (exact: the spacing there is 1), 1032 is
// subtracted exactly, and one fp16 multiply (correctly rounded) applies d.
// out[h] packs K-values 2h (low half) and 2h + 1.
typedef _Float16 kva_half2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void q4_0_f16x8(uint32_t codes, uint16_t d_bits, uint32_t out[4]) {
    const _Float16 d = __builtin_bit_cast(_Float16, d_bits);
    const kva_half2 dd = {d, d};
    const kva_half2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t t = ((codes >> (4 * h)) & 0x000F000Fu) | 0x64006400u;   // 1024 + n, two halves
        const kva_half2 v = (__builtin_bit_cast(kva_half2, t) - off) * dd;
        out[h] = __builtin_bit_cast(uint32_t, v);
    }
}

// Eight q8_0 weights as the fp16 values the MFMA consumes: a chunk of 8
// codes (q8_chunk_pack order and bias) times the fp16 scale d_bits, each
// product rounded once to nearest-even fp16.  One byte permute puts a code
// pair under the exponent byte 0x64, i.e. into the mantissas of two fp16
// values 1024 + (q + 128) (exact: the spacing there is 1); 1152 is
// subtracted exactly, and one fp16 multiply (correctly rounded, so this is
// q8_0_value rounded once) applies d: three instructions per pair.
// out[h] packs K-values 2h (low half) and 2h + 1.
__device__ __forceinline__ void q8_0_f16x8(uint32_t c0, uint32_t c1, uint16_t d_bits, uint32_t out[4]) {
    const _Float16 d = __builtin_bit_cast(_Float16, d_bits);
    const kva_half2 dd = {d, d};
    const kva_half2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        // bytes 4..7 of the permute's input are the codes word, bytes 0..3 the
        // exponent byte: result bytes (code 2 or 3, 0x64, code 0 or 1, 0x64)
        const uint32_t sel = (h & 1) ? 0x00070005u : 0x00060004u;
        const uint32_t t = __builtin_amdgcn_perm(h < 2 ? c0 : c1, 0x64646464u, sel);
        const kva_half2 v = (__builtin_bit_cast(kva_half2, t) - off) * dd;
        out[h] = __builtin_bit_cast(uint32_t, v);
    }
}
// 256x256: 8 waves (2 per SIMD); 128x128: 4 waves; 64xN (calls of at most
// 64 rows): 2 waves of 64 x 32 (N = 64), or of 64 x 64 for SwiGLU (N = 128).
// TILE_128x256: the input GEMM with 16-bit weights only (EPI_INPUT)
enum GemmTile : int { TILE_256x256 = 0, TILE_128x128 = 1, TILE_256x128 = 2, TILE_64xN = 3, TILE_128x256 = 4 };

// The GEMM.  A rows are grouped by 256 like the weight rows (rows >= M of
// the last group are read and dropped).  32-wide K slabs through a ring of
// LDS stages; tiles 256x256 or 128x128.
hipError_t launch_gemm_t32(GemmOperand opd, GemmTile tile, EpiKind epi, const GemmArgs& args,
                           hipStream_t stream);
// The skinny GEMM for calls of at most 32 rows (contexts of at most 32
// tokens per call use it for every trunk GEMM): K split over the waves of a
// workgroup, no LDS ring; split-K across workgroups for EPI_PARTIAL only.
hipError_t launch_gemm_skinny(GemmOperand opd, EpiKind epi, const GemmArgs& args, hipStream_t stream);

// The head GEMM (EPI_HEADS, no split): 256x256 tiles over a whole number of
// rounds of n_cu workgroups, the remaining columns in smaller tiles (128 rows);
// calls of at most 128 rows use one M-tile of 64 or 128 rows.  The first
// min_big 256-column tiles always run 256 columns wide (the fused KV epilogue
// needs a KV head's 256 columns in one workgroup).
hipError_t launch_gemm_heads(GemmOperand opd, const GemmArgs& args, int n_cu, int min_big, hipStream_t stream);

// Folds split-K partials into the residual stream and normalises it:
//   h[r][c] = (add ? h[r][c] : 0) + P_0[r][c] + P_1[r][c] + ... (this order),
//   out[r][c] = 16-bit(h[r][c] / sqrt(mean_c h[r][c]^2 + eps) * g[c]).
// P_s = partials + s * pstride, rows of ldp.  out is in the tiled32_index
// layout (K = cols; cols % 32 == 0).
// With ss (the partials of an EPI_INPUT GEMM; add is then false), the sum
// is then scaled by the input row's 1/RMS:
//   h[r][c] = (P_0[r][c] + P_1[r][c] + ...) * rin[r],
//   rin[r] = 1 / sqrt((ss_0[r] + ss_1[r] + ...) / ss_cols + eps),
// ss_s = ss + s * ss_stride (one value per row, `splits` of them).
hipError_t launch_fold_rmsnorm(float* h, int64_t ldh, bool add, const float* partials, int32_t splits,
                               int64_t pstride, int64_t ldp, const float* g, int32_t rows, int32_t cols,
                               float eps, uint16_t* out, bool bf16, hipStream_t stream,
                               const float* ss = nullptr, int64_t ss_stride = 0, int32_t ss_cols = 0);

// out[tiled32_index(r, c, cols)] = 16-bit(x[r][c]) (fp16 or bf16, nearest
// even); cols % 32 == 0.
hipError_t launch_cast_tiled(const float* x, int64_t ldx, int32_t rows, int32_t cols, uint16_t* out, bool bf16,
                             hipStream_t stream);

// dst[r][c] = src[tiled32_index(r, c, cols)] for r < rows (16-bit values).
hipError_t launch_untile32(const uint16_t* src, uint16_t* dst, int32_t rows, int32_t cols, hipStream_t stream);

// out[tiled32_index(r, c, cols)] = 16-bit(x[r][c] / sqrt(mean_c x[r][c]^2 + eps) * g[c]);
// fp16 or bf16; cols % 32 == 0.
hipError_t launch_rmsnorm_cast(const float* x, int64_t ldx, const float* g, int32_t rows,
                               int32_t cols, float eps, uint16_t* out, bool bf16, hipStream_t stream);

// Block-causal multi-head attention with heads of 128.
//   qk: [n][ld_qk] fp16, Q of head h at columns [h*128, h*128+128), K at k_off + h*128
//   vt: [n_heads*128][ld_vt] fp16, V transposed (vt[c][t])
//   o : fp16 at o[tiled32_index(t, c, ld_o)] (ld_o = n_heads*128, a multiple of 32)
hipError_t launch_attention(const uint16_t* qk, int64_t ld_qk, int32_t k_off, const uint16_t* vt,
                            int64_t ld_vt, uint16_t* o, int64_t ld_o, int32_t n_tokens,
                            int32_t n_heads, int32_t attn_block, hipStream_t stream);

struct KvWriteArgs {
    const float* kv;        // row t: k of the 4 KV heads, then v
    int64_t ld_kv;
    int32_t n_tokens;
    int64_t pos0;
    KvPool pool;
    KvRope rope;
};
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);

// Gated-DeltaNet state update (kva_deltanet.hip).  Key and value heads of
// kDnHeadDim, causal conv of width kDnConv; one launch takes up to
// kMaxDnLayers layers.
constexpr int kDnHeadDim = 128;
constexpr int kDnConv = 4;
constexpr int kMaxDnLayers = 32;

struct DnLayer {
    const float* x;          // [n_tokens][ld]: q|k|v raw, then a (n_v), then b (n_v)
    int64_t ld;
    const float* conv_w;     // [q|k|v channels][kDnConv], 16-byte aligned
    const float* a_log;      // [n_v]
    const float* dt_bias;    // [n_v]
    float* conv_state;       // [kDnConv - 1][q|k|v channels], in/out
    float* state;            // [n_v][kDnHeadDim (v)][kDnHeadDim (k)] fp32, in/out
};

struct DnArgs {
    int32_t n_tokens;
    int32_t n_layers;
    int32_t n_k;             // key heads (q and k)
    int32_t n_v;             // value heads, a multiple of n_k
    DnLayer layer[kMaxDnLayers];
};
hipError_t launch_deltanet_update(const DnArgs& a, hipStream_t stream);

hipError_t launch_dequant_q8_0(const void* blocks, int64_t n_blocks, float* out, hipStream_t stream);
hipError_t launch_dequant_q8_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, hipStream_t stream);
hipError_t launch_check_q8_scale(unsigned long long* counts, hipStream_t stream);
hipError_t launch_dequant_q4_0_f16(const void* blocks, int64_t n_blocks, uint16_t* out, hipStream_t stream);

// n_workgroups x 4 waves, each n_iter x 8 bf16 32x32x16 MFMAs; sink: 256 floats per workgroup.
hipError_t launch_mfma_loop(int32_t n_iter, int32_t n_workgroups, float* sink, hipStream_t stream);

}  // namespace kva
