// Host-side driver of the sanitizer build of the C-ABI layer and the
// rotation-fitting host code (AddressSanitizer + UndefinedBehaviorSanitizer
// on the host code only; no kernel is launched). It calls every entry point
// whose work is host code -- layout geometry, workspace sizing, the
// automatic split choice, argument validation that returns before any
// launch, status strings and the host rotation fit (including calibration
// rows with channels that are zero in every row, and fewer rows than
// channels) -- and checks their results. The kernel launchers are replaced
// by stubs: a launch reached from here is an error.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "rq_internal.h"

namespace rq {
static int launches = 0;
hipError_t launch_decode(const DecodeCall &) { ++launches; return hipErrorNotSupported; }
hipError_t launch_chunk(const ChunkCall &) { ++launches; return hipErrorNotSupported; }
hipError_t launch_encode(const EncodeCall &) { ++launches; return hipErrorNotSupported; }
hipError_t launch_bf16_decode(const Bf16Call &) { ++launches; return hipErrorNotSupported; }
hipError_t launch_bf16_write(int, int, int, uint16_t *, uint16_t *, const uint16_t *, const int64_t *, int,
                             hipStream_t) {
    ++launches;
    return hipErrorNotSupported;
}
hipError_t launch_fit_pass(const FitPass &) { ++launches; return hipErrorNotSupported; }
}  // namespace rq

static int failures = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static rq_layout make(int H, int D, int G, int L, const int *bits, int nblk, int meta, int kv) {
    rq_layout lay;
    memset(&lay, 0, sizeof(lay));
    lay.num_heads = H; lay.head_dim = D; lay.group_size = G; lay.num_loops = L; lay.block_size = 16;
    lay.num_blocks = nblk; lay.meta_dtype = meta; lay.kv_dtype = kv; lay.mode = RQ_MODE_RESIDUAL;
    for (int l = 0; l + 1 < L; ++l) lay.loop_bits[l] = (uint8_t)bits[l];
    return lay;
}

int main() {
    const int b222[3] = {2, 2, 2}, b44222[7] = {4, 4, 2, 2, 2, 2, 2};
    rq_layout ouro = make(16, 128, 128, 4, b222, 300, RQ_DTYPE_F16, RQ_DTYPE_BF16);
    rq_layout hug = make(55, 96, 96, 8, b44222, 5, RQ_DTYPE_F16, RQ_DTYPE_BF16);
    CHECK(rq_layout_check(&ouro) == RQ_OK);
    CHECK(rq_layout_check(&hug) == RQ_OK);
    // slab of the Ouro-like layout: reference 1088 B and three INT2 records of 608 B, K and V each
    CHECK(rq_pool_bytes(&ouro) == (size_t)300 * 16 * 2 * (1088 + 3 * 608));
    CHECK(rq_record_bytes(&ouro, 3) == 1088 && rq_record_bytes(&ouro, 0) == 608);
    CHECK(rq_record_offset(&ouro, 1, 2, 3, 1) == ((int64_t)(1 * 16 + 2) * 5824 + 3 * 1216 + 1088));
    CHECK(rq_record_offset(&ouro, 300, 0, 0, 0) == -1);
    // invalid layouts
    rq_layout bad = ouro;
    bad.head_dim = 80; bad.group_size = 80; CHECK(rq_layout_check(&bad) == RQ_ERR_UNSUPPORTED);
    bad = ouro; bad.group_size = 48; CHECK(rq_layout_check(&bad) == RQ_ERR_SHAPE);
    bad = ouro; bad.loop_bits[1] = 3; CHECK(rq_layout_check(&bad) == RQ_ERR_UNSUPPORTED);
    bad = ouro; bad.num_loops = 17; CHECK(rq_layout_check(&bad) == RQ_ERR_SHAPE);
    CHECK(rq_layout_check(nullptr) == RQ_ERR_NULL);
    CHECK(rq_pool_bytes(&bad) == 0);
    // workspace sizing and the automatic split
    for (int n = 1; n <= 4; ++n) {
        const size_t ws = rq_decode_workspace_bytes(&ouro, n, 16, 2049, 0);
        CHECK(ws > 0);
        CHECK(rq_decode_workspace_bytes(&ouro, n, 16, 2049, 8) > 0);
    }
    const int sp = rq_decode_auto_split_pages(&ouro, 1, 16, 2049);
    CHECK(sp >= 1 && sp <= 64 && sp % 8 == 0);
    CHECK(rq_decode_workspace_bytes(&ouro, 1, 16, 2049, 65) == 0);
    CHECK(rq_bf16_auto_split_pages(16, 16, 2049) >= 1);
    CHECK(rq_bf16_workspace_bytes(16, 128, 16, 2049, 0) > 0);
    CHECK(rq_chunk_workspace_bytes(&ouro, 64, 16, 2049, 0) > 0);
    CHECK(rq_chunk_workspace_bytes(&ouro, 300, 16, 2049, 0) == 0);
    CHECK(rq_fit_workspace_bytes(128) > 0 && rq_fit_workspace_bytes(80) == 0);
    // validation that returns before any launch
    std::vector<uint8_t> host(1 << 16);
    void *p = host.data();
    const float *fp = (const float *)p;
    const int32_t loops[2] = {0, 3}, bad_loops[1] = {4};
    CHECK(rq_decode_attention(&ouro, p, nullptr, 1, p, fp, (int32_t *)p, (int32_t *)p, 1, 1, nullptr, nullptr,
                              0.1f, (float *)p, p, 1 << 16, nullptr) == RQ_ERR_NULL);
    CHECK(rq_decode_attention(&ouro, p, bad_loops, 1, p, fp, (int32_t *)p, (int32_t *)p, 1, 1, nullptr, nullptr,
                              0.1f, (float *)p, p, 1 << 16, nullptr) == RQ_ERR_SHAPE);
    CHECK(rq_decode_attention(&ouro, p, loops, 2, p, fp, (int32_t *)p, (int32_t *)p, 1, 1, p, nullptr, 0.1f,
                              (float *)p, p, 1 << 16, nullptr) == RQ_ERR_NULL);
    CHECK(rq_decode_attention(&ouro, p, loops, 2, p, fp, (int32_t *)p, (int32_t *)p, 1, 1, nullptr, nullptr,
                              NAN, (float *)p, p, 1 << 16, nullptr) == RQ_ERR_SHAPE);
    CHECK(rq_decode_attention(&ouro, p, loops, 2, p, fp, (int32_t *)p, (int32_t *)p, 1, 4096, nullptr, nullptr,
                              0.1f, (float *)p, p, 16, nullptr) == RQ_ERR_WORKSPACE);
    CHECK(rq_decode_attention(&ouro, p, loops, 2, p, fp, (int32_t *)p, (int32_t *)p, 0, 1, nullptr, nullptr,
                              0.1f, (float *)p, p, 16, nullptr) == RQ_OK);   // empty batch: nothing to do
    CHECK(rq_encode_pack(&ouro, p, p, fp, (const int64_t *)p, -1, nullptr) == RQ_ERR_SHAPE);
    CHECK(rq_encode_pack(&ouro, p, p, nullptr, (const int64_t *)p, 4, nullptr) == RQ_ERR_NULL);
    CHECK(rq_chunk_attention(&ouro, p, 0, 300, p, fp, (int32_t *)p, (int32_t *)p, 1, 1, nullptr, nullptr, 0.1f,
                             (float *)p, p, 1 << 16, nullptr, nullptr) == RQ_ERR_UNSUPPORTED);
    CHECK(rq_chunk_attention(&hug, p, 0, 4, p, fp, (int32_t *)p, (int32_t *)p, 1, 1, nullptr, nullptr, 0.1f,
                             (float *)p, p, 1 << 16, nullptr, nullptr) != RQ_OK);
    CHECK(rq_bf16_decode_attention(16, 100, 16, 10, p, p, p, (int32_t *)p, (int32_t *)p, 1, 1, nullptr, nullptr,
                                   0.1f, (float *)p, p, 1 << 16, nullptr) != RQ_OK);
    for (int s = -6; s <= 0; ++s) CHECK(rq_status_string(s) != nullptr && strlen(rq_status_string(s)) > 0);
    CHECK(rq::launches == 0);

    // host rotation fit: full rank, zero channels, fewer rows than channels
    for (int c = 0; c < 3; ++c) {
        const int D = 64, n = c == 2 ? 40 : 300, iters = 2;
        std::vector<float> x((size_t)n * D), r0((size_t)D * D, 0.f), r((size_t)D * D);
        uint32_t s = 12345u + c;
        for (auto &v : x) {
            s = s * 1664525u + 1013904223u;
            v = ((float)(s >> 8) / 16777216.0f - 0.5f) * 0.3f;
        }
        if (c == 1)
            for (int i = 0; i < n; ++i)
                for (int k = 0; k < 4; ++k) x[(size_t)i * D + 7 * k] = 0.f;
        for (int i = 0; i < D; ++i) r0[(size_t)i * D + (i + 1) % D] = 1.f;   // a permutation
        std::vector<double> obj(iters + 1);
        CHECK(rq_fit_rotation(x.data(), n, D, 2, 32, RQ_DTYPE_F16, r0.data(), iters, r.data(), obj.data()) ==
              RQ_OK);
        double worst = 0.0;
        for (int i = 0; i < D; ++i)
            for (int j = 0; j < D; ++j) {
                double d = 0.0;
                for (int k = 0; k < D; ++k) d += (double)r[(size_t)i * D + k] * r[(size_t)j * D + k];
                worst = fmax(worst, fabs(d - (i == j ? 1.0 : 0.0)));
            }
        CHECK(worst < 1e-5);
        for (double o : obj) CHECK(isfinite(o) && o >= 0.0);
    }
    CHECK(rq_fit_rotation(nullptr, 4, 64, 2, 64, 1, nullptr, 1, nullptr, nullptr) == RQ_ERR_NULL);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("host sanitizer driver: all checks passed\n");
    return 0;
}
