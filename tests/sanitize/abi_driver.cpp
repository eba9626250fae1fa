// Drives the C ABI's host-side argument validation over invalid and edge arguments, for a
// build of the library's host code with AddressSanitizer and UndefinedBehaviorSanitizer (test
// infrastructure). Every call here returns before any HIP call, so no GPU is needed. Exit
// status 0 and "abi driver: ok" when nothing fired and every status is as expected.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "hqq.h"

static int failures = 0;
static void expect(bool ok, const char *what)
{
    if (!ok) {
        std::fprintf(stderr, "unexpected: %s (%s)\n", what, hqq_last_error());
        ++failures;
    }
}

static hqq_job job()
{
    hqq_job j{};
    j.W = reinterpret_cast<void *>(0x1000);
    j.rows = 64;
    j.cols = 256;
    j.nbits = 4;
    j.group_size = 64;
    j.axis = 1;
    j.p = 0.7f;
    j.beta = 1.0f;
    j.kappa = 1.01f;
    j.iters = 20;
    j.early_stop = 1;
    j.zero_bits = 8;
    j.packed = reinterpret_cast<void *>(0x2000);
    j.scale = reinterpret_cast<void *>(0x3000);
    j.zero = reinterpret_cast<void *>(0x4000);
    j.zero_meta = reinterpret_cast<void *>(0x5000);
    return j;
}

int main()
{
    const int64_t big = int64_t(1) << 40;
    for (int nbits = -1; nbits <= 9; ++nbits)
        for (int64_t n : {int64_t(-5), int64_t(0), int64_t(1), int64_t(10), int64_t(11), big})
            (void)hqq_packed_bytes(n, nbits);
    expect(hqq_packed_bytes(11, 3) == 8, "packed bytes 3-bit");

    hqq_job bad[16];
    for (auto &b : bad) b = job();
    bad[0].nbits = 5;
    bad[1].axis = 2;
    bad[2].group_size = 0;
    bad[3].p = std::numeric_limits<float>::quiet_NaN();
    bad[4].beta = -1.0f;
    bad[5].iters = 1000;
    bad[6].zero_bits = 3;
    bad[7].W = nullptr;
    bad[8].rows = -3;
    bad[9].rows = big;
    bad[9].cols = big;
    bad[10].cols = 100;
    bad[11].W = reinterpret_cast<void *>(0x1001);
    bad[12].zero_meta = nullptr;
    bad[13].rows = int64_t(1) << 20;
    bad[13].cols = int64_t(1) << 18;
    bad[14].early_stop = 7;
    bad[15].kappa = std::numeric_limits<float>::infinity();
    for (auto &b : bad) {
        expect(hqq_workspace_bytes(&b, 1) == SIZE_MAX, "workspace of an invalid job");
        expect(hqq_quantize_batch(&b, 1, nullptr, 0, nullptr) != HQQ_OK, "invalid job accepted");
        expect(hqq_batch_check(&b, 1, nullptr, 0, nullptr) != HQQ_OK, "check of an invalid job");
    }
    hqq_job ok[3] = {job(), job(), job()};
    ok[1].nbits = 3;
    ok[2].axis = 0;
    const size_t need = hqq_workspace_bytes(ok, 3);
    expect(need > 0 && need != SIZE_MAX && need % 256 == 0, "workspace of valid jobs");
    expect(hqq_quantize_batch(ok, 3, nullptr, 0, nullptr) == HQQ_ERR_WORKSPACE, "no workspace");
    expect(hqq_quantize_batch(ok, 3, reinterpret_cast<void *>(0x10010), need, nullptr) ==
               HQQ_ERR_ARG, "misaligned workspace");
    expect(hqq_quantize_batch(nullptr, 2, nullptr, 0, nullptr) == HQQ_ERR_ARG, "null jobs");
    expect(hqq_quantize_batch(ok, -1, nullptr, 0, nullptr) == HQQ_ERR_ARG, "negative count");
    expect(hqq_streamed_workspace_bytes(ok, 3, 64) == SIZE_MAX, "staging too small");
    expect(hqq_quantize_streamed(ok, 3, nullptr, 64, nullptr, 0, nullptr, nullptr) ==
               HQQ_ERR_WORKSPACE, "streamed with tiny staging");
    expect(hqq_quantize_noalloc(nullptr, 64, 256, 4, 64, 1, 0.7f, 1.0f, 1.01f, 20, 1, 16,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) ==
               HQQ_ERR_ARG, "noalloc null W");
    expect(hqq_quantize_noalloc(reinterpret_cast<void *>(0x1000), 8192, 8192, 4, 64, 0, 0.7f,
                                1.0f, 1.01f, 20, 1, 16, reinterpret_cast<void *>(0x2000),
                                reinterpret_cast<void *>(0x3000),
                                reinterpret_cast<void *>(0x4000), nullptr, nullptr,
                                nullptr) == HQQ_ERR_WORKSPACE, "noalloc too large");
    expect(hqq_dequantize(nullptr, nullptr, nullptr, nullptr, 8, 64, 4, 64, 1, 16, nullptr,
                          nullptr) == HQQ_ERR_ARG, "dequantize nulls");
    expect(hqq_dequantize(nullptr, nullptr, nullptr, nullptr, 8, 64, 6, 64, 1, 16, nullptr,
                          nullptr) == HQQ_ERR_ARG, "dequantize nbits");
    expect(hqq_gemm(nullptr, 4, nullptr, nullptr, nullptr, nullptr, 8, 64, 4, 64, 16, nullptr,
                    nullptr, 0, nullptr) == HQQ_ERR_ARG, "gemm nulls");
    expect(hqq_gemm(nullptr, -1, nullptr, nullptr, nullptr, nullptr, 8, 64, 4, 64, 16, nullptr,
                    nullptr, 0, nullptr) == HQQ_ERR_ARG, "gemm M");
    expect(hqq_gemm_f16(nullptr, 4, nullptr, 8, 12, nullptr, nullptr) == HQQ_ERR_ARG, "gemm_f16 K");
    expect(hqq_pack(nullptr, 10, 4, nullptr, nullptr) == HQQ_ERR_ARG, "pack nulls");
    expect(hqq_unpack(nullptr, 10, 7, nullptr, nullptr) == HQQ_ERR_ARG, "unpack nbits");
    expect(hqq_requant_scales(nullptr, 100, 100, nullptr, nullptr, nullptr) == HQQ_ERR_ARG,
           "scale group");
    expect(hqq_dequantize_scales(nullptr, nullptr, -1, 128, nullptr, nullptr) == HQQ_ERR_ARG,
           "scale count");
    expect(hqq_gemm_workspace_bytes(1000, 1 << 20, 1 << 20) > 0, "gemm workspace");
    for (int s = 0; s <= 7; ++s) (void)hqq_status_string(static_cast<hqq_status>(s));
    if (failures) return 1;
    std::printf("abi driver: ok\n");
    return 0;
}
