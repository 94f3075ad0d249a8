// Exercise of the library's host-side logic (linear_attention_amd/csrc/
// host_logic.h: argument checks, ALiBi slopes, the sequence-segment plan and
// its workspace size, the checks of device metadata) for the sanitizer
// builds of the CPU test suite.  Built with g++ -fsanitize=address,undefined;
// any report fails the test.  Arguments sweep the valid ranges and their
// edges: zero and negative sizes, int32 limits, empty batches, out-of-range
// and duplicate slots, malformed offsets and parents.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "host_logic.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main() {
    using namespace la;
    alignas(16) static char buf[64];
    const void *p = buf, *mis = buf + 8;
    const float *f = reinterpret_cast<const float *>(buf);
    const int32_t *ip = reinterpret_cast<const int32_t *>(buf);

    // argument checks
    const int sizes[] = {-2147483647 - 1, -1, 0, 1, 2, 3, 64, 65, 128, 4096, 2147483647};
    int ok = 0;
    for (int batch : sizes)
        for (int H : sizes)
            for (int HK : {-1, 0, 1, 2, 3, 64})
                for (int d : {-1, 0, 32, 64, 100, 128, 256})
                    for (int64_t T : {int64_t(-1), int64_t(0), int64_t(5), int64_t(1) << 31, int64_t(1) << 40})
                        for (int64_t P : {int64_t(0), int64_t(1), int64_t(4096), int64_t(1) << 33}) {
                            const la_status s = common_checks(p, p, p, LA_DTYPE_BF16, T, batch, H, HK, d, f, P, ip,
                                                              f, p);
                            ok += s == LA_OK;
                        }
    CHECK(ok > 0);
    CHECK(common_checks(mis, p, p, LA_DTYPE_F32, 5, 1, 4, 4, 128, f, 4, ip, f, p) == LA_ERR_INVALID_ARG);
    CHECK(common_checks(p, p, p, static_cast<la_dtype>(7), 5, 1, 4, 4, 128, f, 4, ip, f, p) == LA_ERR_UNSUPPORTED);
    CHECK(common_checks(nullptr, nullptr, nullptr, LA_DTYPE_BF16, 0, 0, 4, 4, 64, f, 4, nullptr, f, nullptr) == LA_OK);

    // slopes
    std::vector<float> sl(5000);
    for (int H = 1; H <= 5000; H += (H < 300 ? 1 : 97))
        for (int L : {1, 2, 4, 48})
            for (int l = 0; l < L; l += (L > 4 ? 11 : 1)) {
                CHECK(alibi_slopes(H, l, L, sl.data()) == LA_OK);
                for (int h = 0; h < H; ++h) CHECK(sl[h] > 0.f && sl[h] <= 1.00001f);
            }
    CHECK(alibi_slopes(0, 0, 1, sl.data()) == LA_ERR_INVALID_ARG);
    CHECK(alibi_slopes(4, 1, 1, sl.data()) == LA_ERR_INVALID_ARG);
    CHECK(alibi_slopes(4, 0, 1, nullptr) == LA_ERR_INVALID_ARG);

    // segment plan: bounded segment counts and exact workspace sizes
    for (int cus : {1, 80, 256, 304, 1024})
        for (int batch : {-1, 0, 1, 2, 3, 8, 64, 65536, 2147483647})
            for (int H : {-5, 0, 1, 2, 8, 64, 2147483647})
                for (int d : {32, 64, 128})
                    for (int L : {-1, 0, 8191, 8192, 131072, 2147483647})
                        for (bool track : {false, true})
                            for (int cap : {-3, 1, 2, 8, 100}) {
                                const SegmentPlan pl = plan_segments(cus, batch, H, d, L, track, cap);
                                CHECK(pl.segments >= 1 && pl.segments <= kMaxSegments);
                                if (pl.segments == 1) {
                                    CHECK(pl.workspace_bytes == 0);
                                    continue;
                                }
                                CHECK(!track && L >= kMinSplitTokens && cap >= 2);
                                CHECK(pl.subsegs >= 1 && pl.subsegs <= kMaxSubsegs);
                                const size_t pairs = static_cast<size_t>(batch) * H;
                                const size_t slices = pairs * (pl.segments - 1) * pl.subsegs + pairs * pl.segments;
                                CHECK(pl.workspace_bytes == slices * d * d * sizeof(float));
                            }

    // on a 256-CU part every split fits the static scratch of la_prefill_noalloc
    size_t most = 0;
    for (int batch = 1; batch <= 64; ++batch)
        for (int H = 1; H <= 64; ++H)
            for (int d : {64, 128}) {
                const SegmentPlan pl = plan_segments(256, batch, H, d, 1 << 20, false, kMaxSegments);
                most = pl.workspace_bytes > most ? pl.workspace_bytes : most;
            }
    CHECK(most > 0 && most <= LA_NOALLOC_SCRATCH_BYTES);
    std::printf("largest split workspace on 256 CUs: %zu bytes\n", most);

    // metadata checks
    const int32_t cu_ok[4] = {0, 3, 3, 10}, cu_dec[4] = {0, 5, 4, 10}, cu_big[4] = {0, 3, 3, 2147483647};
    const int32_t slots[3] = {2, 0, 5}, dup[3] = {2, 0, 2}, neg[3] = {2, -1, 5}, far[3] = {2, 0, 2147483647};
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, slots, 6, nullptr, nullptr, nullptr) == LA_OK);
    CHECK(check_metadata(cu_ok, 3, 10, 6, 0, slots, 6, nullptr, nullptr, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_dec, 3, 10, 7, 0, slots, 6, nullptr, nullptr, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_big, 3, 10, 7, 0, slots, 6, nullptr, nullptr, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, dup, 6, nullptr, nullptr, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, neg, 6, nullptr, nullptr, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, far, 6, nullptr, nullptr, nullptr) == LA_ERR_INVALID_ARG);
    const int32_t tl[3] = {3, 0, 7}, tl_bad[3] = {4, 0, 7}, ts[3] = {1, -1, 3}, ts_dup[3] = {1, 1, 3},
                  ts_act[3] = {1, -1, 5};
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, slots, 6, tl, ts, nullptr) == LA_OK);
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, slots, 6, tl_bad, ts, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, slots, 6, tl, ts_dup, nullptr) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(cu_ok, 3, 10, 7, 0, slots, 6, tl, ts_act, nullptr) == LA_ERR_INVALID_ARG);
    const int32_t par_ok[6] = {-1, 0, -1, -1, 0, 1}, par_bad[6] = {-1, 1, -1, -1, 0, 1};
    CHECK(check_metadata(nullptr, 2, 6, 3, 3, slots, 6, nullptr, nullptr, par_ok) == LA_OK);
    CHECK(check_metadata(nullptr, 2, 6, 3, 3, slots, 6, nullptr, nullptr, par_bad) == LA_ERR_INVALID_ARG);
    CHECK(check_metadata(nullptr, 2, 6, 3, 0, slots, 6, nullptr, nullptr, par_ok) == LA_ERR_INVALID_ARG);
    const int32_t cu0[1] = {0};
    CHECK(check_metadata(cu0, 0, 0, 0, 0, nullptr, 1, nullptr, nullptr, nullptr) == LA_OK);
    std::puts("host driver ok");
    return 0;
}
