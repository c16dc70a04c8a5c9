// Drives the host-side entry points of the HIP library that need no GPU
// (blob sizes, the host repack at every weight format, argument validation
// of layer creation, the allocation cap), for a build whose host code runs
// under AddressSanitizer and UndefinedBehaviorSanitizer.  Exit status 0
// means every call returned its documented code.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "coli_moe.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main() {
    uint32_t state = 777u;
    auto next = [&] { state = state * 1664525u + 1013904223u; return state >> 8; };
    const int shapes[][2] = {{128, 128}, {512, 384}, {384, 640}};
    for (const auto &hw : shapes) {
        for (int g : {32, 64}) {
            for (int b : {4, 8}) {
                const size_t n = coli_expert_blob_bytes(hw[0], hw[1], g, b);
                CHECK(n > 0);
                std::vector<unsigned char> src(n), dst(n);
                for (auto &v : src) v = static_cast<unsigned char>(next());
                CHECK(coli_expert_repack(src.data(), dst.data(), hw[0], hw[1], g, b) == COLI_OK);
            }
        }
    }
    std::vector<unsigned char> buf(4096);
    CHECK(coli_expert_repack(buf.data(), buf.data(), 96, 128, 32, 4) == COLI_E_INVALID);
    CHECK(coli_expert_repack(nullptr, buf.data(), 128, 128, 32, 4) == COLI_E_INVALID);
    CHECK(coli_expert_blob_bytes(128, 128, 16, 4) == 0);

    coli_moe_dims d{256, 128, 16, 4, 0, 8, COLI_ACT_F32, 32, 4};
    coli_layer *L = nullptr;
    d.top_k = 40;
    CHECK(coli_layer_create(&d, 0, &L) == COLI_E_INVALID && L == nullptr);
    d.top_k = 4;
    d.hidden = 192;
    CHECK(coli_layer_create(&d, 0, &L) == COLI_E_UNSUPPORTED && L == nullptr);
    d.hidden = 256;
    CHECK(coli_set_alloc_limit(1000) == COLI_OK);
    CHECK(coli_layer_create(&d, 0, &L) == COLI_E_NOMEM && L == nullptr);
    CHECK(coli_set_alloc_limit(-1) == COLI_OK);
    CHECK(coli_set_alloc_limit(-5) == COLI_E_INVALID);
    CHECK(coli_alloc_bytes() == 0);
    CHECK(coli_router_set(nullptr, nullptr, nullptr) == COLI_E_INVALID);
    CHECK(coli_last_error(nullptr) != nullptr);
    std::printf("abi driver ok\n");
    return 0;
}
