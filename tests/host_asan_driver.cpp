// Host-side driver for the AddressSanitizer check of libbakron's host code.
//
// It calls every entry point along the paths that finish on the host: the
// workspace-size queries, the schedule summary and the full step list of the
// recursion plan (many shapes, both product orders, concurrent first calls
// for one shape from several threads), and the argument checks that reject a
// call before it touches a device (NULL or misaligned pointers, bad shapes,
// quantizers and flags, small workspaces).  No GPU is needed: no call here
// reaches a HIP runtime function.  Built against a library whose host code
// carries -fsanitize=address, any out-of-bounds access or use-after-free in
// those paths aborts the run with a report.
//
// Exit status 0 when every call returned what the C ABI documents.
#include <bakron.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

static int g_fail = 0;

#define CHECK(cond)                                                             \
    do {                                                                        \
        if (!(cond)) {                                                          \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++g_fail;                                                           \
        }                                                                       \
    } while (0)

// Walks the step list of one plan and checks the fields the header defines.
static void plan_fields(int64_t m, int64_t n, int32_t flags) {
    int64_t count = -1;
    CHECK(bakron_schedule_plan(m, n, flags, nullptr, 0, &count) == BAKRON_OK);
    CHECK(count >= 1);
    if (count < 1) return;
    // too small an array is refused without a write
    std::vector<int32_t> small(16 * (count - 1) + 1, 7);
    int64_t c2 = -1;
    CHECK(bakron_schedule_plan(m, n, flags, small.data(), count - 1, &c2) ==
          BAKRON_ERR_INVALID_ARG);
    for (int32_t v : small) CHECK(v == 7);
    std::vector<int32_t> ops(16 * count);
    CHECK(bakron_schedule_plan(m, n, flags, ops.data(), count, &c2) == BAKRON_OK && c2 == count);
    const int64_t D = (m + 63) / 64 + (n + 63) / 64 - 1;
    int64_t leaves = 0;
    for (int64_t k = 0; k < count; ++k) {
        const int32_t *o = &ops[16 * k];
        CHECK(o[0] >= 0 && o[0] <= 3);
        if (o[0] == 0) {
            CHECK(o[3] == leaves);  // leaves in diagonal order
            ++leaves;
        } else if (o[0] == 1) {
            CHECK(o[3] >= 0 && o[5] >= 2 && o[6] >= 1 && o[6] < o[5] && o[3] + o[5] <= D);
            CHECK(o[8] == 0 || o[8] == 1);
        } else {
            CHECK(o[2] >= 0);
        }
    }
    CHECK(leaves == D);
}

static void shapes_and_orders() {
    const int64_t shapes[][2] = {{1, 1},      {1, 300},     {300, 1},    {63, 65},
                                 {64, 64},    {65, 127},    {129, 193},  {1024, 1024},
                                 {1536, 1024}, {1024, 3008}, {4096, 4096}, {11008, 4096},
                                 {4096, 14336}, {64, 20000}, {20000, 64}};
    for (auto &s : shapes) {
        for (int32_t order = 0; order <= 3; ++order) {
            double info[15];
            std::memset(info, 0, sizeof info);
            CHECK(bakron_schedule_info(s[0], s[1], order, info) == BAKRON_OK);
            CHECK(info[0] == 64.0 && info[1] >= 1.0);
            CHECK(info[4] == 1.0 || info[4] == 2.0);
            plan_fields(s[0], s[1], order);
        }
        for (int32_t kind = 0; kind <= 2; ++kind)
            for (int32_t bits = 2; bits <= 8; ++bits) {
                const size_t q = bakron_quantize_workspace_size(s[0], s[1], kind, bits);
                const size_t a = bakron_quantize_antidiag_workspace_size(s[0], s[1], kind, bits);
                // a workspace size is 0 exactly for the quantizers the library refuses
                CHECK((q == 0) == (a == 0));
            }
    }
    double info[15];
    CHECK(bakron_schedule_info(0, 4, 0, info) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_schedule_info(4, -1, 0, info) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_schedule_info(4, 4, 0, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_schedule_info((int64_t)1 << 21, 4, 0, info) == BAKRON_ERR_INVALID_ARG);
    int64_t count;
    CHECK(bakron_schedule_plan(4, 4, 0, nullptr, 0, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_schedule_plan(0, 4, 0, nullptr, 0, &count) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize_workspace_size(0, 4, 0, 4) == 0);
    CHECK(bakron_quantize_workspace_size(4, 4, 0, 9) == 0);
    CHECK(bakron_hessian_workspace_size(8192, 4096) == 0);  // the Gram product needs none
    CHECK(bakron_factor_workspace_size(4096) > 0);
}

// Several threads ask for the same shapes' plans at once: the per-shape
// plan cache is built once and read by all.
static void concurrent_plans() {
    const int64_t shapes[][2] = {{2048, 2048}, {2048, 3072}, {3072, 2048}, {640, 4160}};
    std::vector<std::thread> th;
    for (int t = 0; t < 8; ++t)
        th.emplace_back([&shapes, t] {
            for (int r = 0; r < 3; ++r)
                for (auto &s : shapes) {
                    double info[15];
                    CHECK(bakron_schedule_info(s[0], s[1], (t + r) % 3, info) == BAKRON_OK);
                    plan_fields(s[0], s[1], (t + r) % 3);
                }
        });
    for (auto &x : th) x.join();
}

// Calls that are rejected on the host, before any device access.
static void argument_errors() {
    void *fake = reinterpret_cast<void *>(4096);
    const float *F = static_cast<const float *>(fake);
    float *Fo = static_cast<float *>(fake);
    int8_t *C = static_cast<int8_t *>(fake);
    CHECK(bakron_quantize(nullptr, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr,
                          nullptr, 0, fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(std::strstr(bakron_last_error(), "non-NULL") != nullptr);
    CHECK(bakron_quantize(F, 0, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                          fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize(F, 4, 4, F, F, 0, 6, C, Fo, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                          fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize(F, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr, nullptr,
                          0x80, fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize(F, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr, nullptr,
                          0x20 | 0x40, fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize(F, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                          fake, 16, nullptr) == BAKRON_ERR_WORKSPACE);
    CHECK(bakron_quantize(F, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                          reinterpret_cast<void *>(4096 + 8), 1 << 30, nullptr) ==
          BAKRON_ERR_WORKSPACE);
    CHECK(bakron_quantize_noalloc(F, 4096, 4096, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, 0, nullptr) == BAKRON_ERR_WORKSPACE);
    CHECK(bakron_quantize_noalloc(F, 64, 64, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, 0x4, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize_antidiag(nullptr, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr,
                                   nullptr, fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_quantize_antidiag(F, 4, 4, F, F, 0, 4, C, Fo, nullptr, nullptr, nullptr, nullptr,
                                   fake, 8, nullptr) == BAKRON_ERR_WORKSPACE);
    CHECK(bakron_hessian(nullptr, 4, 4, 0.01f, Fo, nullptr, 0, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_hessian(F, 4, 4, -1.0f, Fo, nullptr, 0, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_factor(F, 0, Fo, nullptr, fake, 1 << 20, nullptr) == BAKRON_ERR_INVALID_ARG);
    CHECK(bakron_factor(F, 8, Fo, nullptr, fake, 8, nullptr) == BAKRON_ERR_WORKSPACE);
    double ph[10];
    CHECK(bakron_last_phase_ms(ph) == BAKRON_ERR_INVALID_ARG);
    for (int32_t s = -2; s <= 12; ++s) CHECK(bakron_status_string(s) != nullptr);
    // the error message belongs to the calling thread
    std::thread([] {
        CHECK(bakron_schedule_info(0, 0, 0, nullptr) == BAKRON_ERR_INVALID_ARG);
        CHECK(std::strlen(bakron_last_error()) > 0);
    }).join();
}

int main() {
    shapes_and_orders();
    concurrent_plans();
    argument_errors();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("host checks passed\n");
    return 0;
}
