// Host-only exercise of the C ABI for a sanitizer build (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host code of the runtime): config
// validation, the head plan, weight packing for every device layout, the
// fp16 conversion, status strings.  Needs no GPU.  Exits non-zero on a wrong
// status; the sanitizers abort on a memory or UB error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "kva.h"

static int failures = 0;
#define EXPECT(cond)                                                         \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, kva_last_error()); \
            ++failures;                                                      \
        }                                                                    \
    } while (0)

static std::vector<kva_head_desc> late_heads(bool drafters) {
    std::vector<kva_head_desc> h;
    for (int layer = 32; layer < 64; ++layer) {
        if (layer % 4 == 3) h.push_back({KVA_HEAD_ATTN, layer, 2048});
        else h.push_back({KVA_HEAD_DELTANET, layer, 10336});
    }
    if (drafters)
        for (int layer : {34, 48, 62, 64}) h.push_back({KVA_HEAD_DRAFT, layer, 5120});
    return h;
}

static kva_config make_cfg(std::vector<kva_head_desc>& heads, int d, int F) {
    kva_config c{};
    c.n_in = 5120; c.d_model = d; c.n_blocks = 3; c.n_heads = d / 128; c.head_dim = 128; c.d_ffn = F;
    c.attn_block = 1024; c.max_tokens = 1024; c.eps = 1e-6f; c.weight_dtype = KVA_DTYPE_BF16;
    c.has_head_bias = 1; c.n_out_heads = (int32_t)heads.size(); c.out_heads = heads.data();
    return c;
}

int main() {
    // validation
    auto h2 = late_heads(false), h3 = late_heads(true);
    kva_config r2 = make_cfg(h2, 2560, 7040), r3 = make_cfg(h3, 3072, 8448);
    EXPECT(kva_validate_config(&r2) == KVA_OK);
    EXPECT(kva_validate_config(&r3) == KVA_OK);
    kva_config bad = r2; bad.head_dim = 64;
    EXPECT(kva_validate_config(&bad) == KVA_ERR_SHAPE);
    bad = r2; bad.n_out_heads = 0;
    EXPECT(kva_validate_config(&bad) == KVA_ERR_SHAPE);
    bad = r2; bad.out_heads = nullptr;
    EXPECT(kva_validate_config(&bad) == KVA_ERR_ARG);
    EXPECT(kva_validate_config(nullptr) == KVA_ERR_ARG);

    // head plan: query the width, then a short and a full buffer
    for (kva_config* c : {&r2, &r3}) {
        int32_t n = 0;
        EXPECT(kva_debug_head_plan(c, &n, nullptr, nullptr, 0) == KVA_OK);
        std::vector<int32_t> head(n), idx(n);
        EXPECT(kva_debug_head_plan(c, &n, head.data(), idx.data(), n - 1) == KVA_ERR_SHAPE);
        EXPECT(kva_debug_head_plan(c, &n, head.data(), idx.data(), n) == KVA_OK);
        int64_t real = 0;
        for (int32_t i = 0; i < n; ++i) real += head[i] >= 0;
        int64_t want = 0;
        for (int i = 0; i < c->n_out_heads; ++i) want += c->out_heads[i].out_dim;
        EXPECT(real == want);
    }

    // fp16 conversion, including non-finite, overflow and subnormal inputs
    std::vector<float> f = {0.f, -0.f, 1.f, 65504.f, 65519.f, 1e-8f, 6e-5f, INFINITY, -INFINITY, NAN};
    std::vector<uint16_t> h(f.size());
    EXPECT(kva_debug_host_to_f16(f.data(), KVA_DTYPE_F32, (int64_t)f.size(), h.data()) == KVA_OK);
    f.push_back(70000.f);
    h.resize(f.size());
    EXPECT(kva_debug_host_to_f16(f.data(), KVA_DTYPE_F32, (int64_t)f.size(), h.data()) == KVA_ERR_RANGE);

    // packing into every layout, ragged row counts, exact and short buffers
    std::mt19937 rng(7);
    for (int rows : {1, 200, 256, 300}) {
        for (int K : {32, 96, 160}) {
            const int rpad = (rows + 255) / 256 * 256;
            std::vector<float> w32((size_t)rows * K);
            for (float& v : w32) v = (float)((int)(rng() % 2001) - 1000) * 1e-4f;
            for (int target : {0, 1}) {
                std::vector<uint8_t> out((size_t)rpad * K * 2);
                EXPECT(kva_debug_pack_weight(w32.data(), KVA_DTYPE_F32, rows, K, target, out.data(),
                                             (int64_t)out.size(), nullptr, 0) == KVA_OK);
                EXPECT(kva_debug_pack_weight(w32.data(), KVA_DTYPE_F32, rows, K, target, out.data(),
                                             (int64_t)out.size() - 1, nullptr, 0) == KVA_ERR_SHAPE);
            }
            const int nb = K / 32;
            std::vector<uint8_t> q8((size_t)rows * nb * 34), q4((size_t)rows * nb * 18);
            for (int r = 0; r < rows; ++r)
                for (int b = 0; b < nb; ++b) {
                    const uint16_t d = 0x1400;   // 2^-10
                    std::memcpy(&q8[((size_t)r * nb + b) * 34], &d, 2);
                    std::memcpy(&q4[((size_t)r * nb + b) * 18], &d, 2);
                    for (int j = 0; j < 32; ++j) q8[((size_t)r * nb + b) * 34 + 2 + j] = (uint8_t)(rng() & 0xFF);
                    for (int j = 0; j < 16; ++j) q4[((size_t)r * nb + b) * 18 + 2 + j] = (uint8_t)(rng() & 0xFF);
                }
            std::vector<uint8_t> out8((size_t)rpad * K), out4((size_t)rpad * K / 2);
            std::vector<uint16_t> sc((size_t)rpad * nb);
            EXPECT(kva_debug_pack_weight(q8.data(), KVA_DTYPE_Q8_0, rows, K, 2, out8.data(), (int64_t)out8.size(),
                                         sc.data(), (int64_t)sc.size()) == KVA_OK);
            EXPECT(kva_debug_pack_weight(q8.data(), KVA_DTYPE_Q8_0, rows, K, 2, out8.data(), (int64_t)out8.size(),
                                         sc.data(), (int64_t)sc.size() - 1) == KVA_ERR_SHAPE);
            EXPECT(kva_debug_pack_weight(q4.data(), KVA_DTYPE_Q4_0, rows, K, 3, out4.data(), (int64_t)out4.size(),
                                         sc.data(), (int64_t)sc.size()) == KVA_OK);
            EXPECT(kva_debug_pack_weight(q4.data(), KVA_DTYPE_Q4_0, rows, K, 2, out8.data(), (int64_t)out8.size(),
                                         sc.data(), (int64_t)sc.size()) == KVA_ERR_DTYPE);
            // an overflowing q8_0 scale
            const uint16_t big = 0x7BFF;
            std::memcpy(&q8[0], &big, 2);
            q8[2] = 0x81;   // code -127
            EXPECT(kva_debug_pack_weight(q8.data(), KVA_DTYPE_Q8_0, rows, K, 2, out8.data(), (int64_t)out8.size(),
                                         sc.data(), (int64_t)sc.size()) == KVA_ERR_RANGE);
        }
    }
    EXPECT(kva_debug_pack_weight(nullptr, KVA_DTYPE_F32, 1, 32, 0, nullptr, 0, nullptr, 0) == KVA_ERR_ARG);
    EXPECT(kva_debug_pack_weight(f.data(), KVA_DTYPE_F32, 1, 33, 0, h.data(), 1 << 20, nullptr, 0) == KVA_ERR_SHAPE);

    // statuses, NULL safety
    for (int s = 0; s <= 7; ++s) EXPECT(std::strncmp(kva_status_str((kva_status)s), "KVA_", 4) == 0);
    EXPECT(kva_destroy(nullptr) == KVA_OK);
    EXPECT(kva_project_ubatch(nullptr, nullptr, 1, nullptr, nullptr) == KVA_ERR_ARG);
    EXPECT(kva_get_stats(nullptr, nullptr) == KVA_ERR_ARG);

    if (failures) {
        std::fprintf(stderr, "%d failure(s)\n", failures);
        return 1;
    }
    std::printf("abi host checks ok\n");
    return 0;
}
