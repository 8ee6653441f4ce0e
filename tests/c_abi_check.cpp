// c_abi_check.cpp -- drives libgemm_bt.so through include/gemm_bt.h alone: no
// Python, no PyTorch, device memory from hipMalloc.  Expected values are closed
// forms of C = A * B^T (all-ones operands give K in every entry; an identity B
// gives A back), so nothing here recomputes the product.  Exit status 0 and a
// line ending in "ok" mean every check passed.  Without a HIP device it checks
// that the library reports GEMM_BT_ERR_NO_DEVICE instead.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gemm_bt.h"

#define REQUIRE(cond)                                                        \
    do {                                                                     \
        if (!(cond)) {                                                       \
            std::printf("c_abi_check FAILED: %s (line %d)\n", #cond, __LINE__); \
            return 1;                                                        \
        }                                                                    \
    } while (0)

// bf16 bits of a small integer (exact: the low 16 bits of its float are zero)
static uint16_t bf16_of(int v) {
    const float f = (float)v;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

int main() {
    REQUIRE(gemm_bt_version() >= 100);
    REQUIRE(gemm_bt_status_string(GEMM_BT_ERR_UNSUPPORTED) != nullptr);
    // argument errors come back before any device is touched
    REQUIRE(gemm_bt((void*)16, (void*)16, (void*)16, -1, 4, 4, GEMM_BT_BF16, GEMM_BT_F32, nullptr) ==
            GEMM_BT_ERR_INVALID_VALUE);
    REQUIRE(gemm_bt((void*)16, (void*)16, (void*)16, 4, 4, 4, 99, GEMM_BT_F32, nullptr) == GEMM_BT_ERR_UNSUPPORTED);

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) {
        (void)hipGetLastError();
        REQUIRE(gemm_bt((void*)256, (void*)256, (void*)256, 4, 4, 4, GEMM_BT_BF16, GEMM_BT_F32, nullptr) ==
                GEMM_BT_ERR_NO_DEVICE);
        std::printf("c_abi_check no-device ok\n");
        return 0;
    }

    // all-ones: every entry is K exactly (f32 output), plain and batched with a shared B
    const int M = 96, N = 80, K = 200, Z = 3;
    std::vector<uint16_t> a((size_t)Z * M * K, bf16_of(1)), b((size_t)N * K, bf16_of(1));
    std::vector<float> c((size_t)Z * M * N, -1.0f);
    void *dA, *dB, *dC;
    REQUIRE(hipMalloc(&dA, a.size() * 2) == hipSuccess);
    REQUIRE(hipMalloc(&dB, b.size() * 2) == hipSuccess);
    REQUIRE(hipMalloc(&dC, c.size() * 4) == hipSuccess);
    REQUIRE(hipMemcpy(dA, a.data(), a.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
    REQUIRE(hipMemcpy(dB, b.data(), b.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
    REQUIRE(gemm_bt(dA, dB, dC, M, N, K, GEMM_BT_BF16, GEMM_BT_F32, nullptr) == GEMM_BT_OK);
    REQUIRE(hipDeviceSynchronize() == hipSuccess);
    REQUIRE(hipMemcpy(c.data(), dC, (size_t)M * N * 4, hipMemcpyDeviceToHost) == hipSuccess);
    for (int i = 0; i < M * N; ++i) REQUIRE(c[i] == (float)K);
    REQUIRE(gemm_bt_batched(dA, dB, dC, Z, M, N, K, (int64_t)M * K, 0, (int64_t)M * N, GEMM_BT_BF16, GEMM_BT_F32,
                            nullptr) == GEMM_BT_OK);
    REQUIRE(hipDeviceSynchronize() == hipSuccess);
    REQUIRE(hipMemcpy(c.data(), dC, c.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
    for (size_t i = 0; i < c.size(); ++i) REQUIRE(c[i] == (float)K);

    // identity B (N = K): C = A bit for bit (bf16 output)
    const int M2 = 70, K2 = 64;
    std::vector<uint16_t> a2((size_t)M2 * K2), id((size_t)K2 * K2, 0), c2((size_t)M2 * K2, 0xFFFF);
    for (int i = 0; i < M2; ++i)
        for (int k = 0; k < K2; ++k) a2[(size_t)i * K2 + k] = bf16_of((i * 7 + k * 3) % 9 - 4);
    for (int k = 0; k < K2; ++k) id[(size_t)k * K2 + k] = bf16_of(1);
    REQUIRE(hipMemcpy(dA, a2.data(), a2.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
    REQUIRE(hipMemcpy(dB, id.data(), id.size() * 2, hipMemcpyHostToDevice) == hipSuccess);
    REQUIRE(gemm_bt(dA, dB, dC, M2, K2, K2, GEMM_BT_BF16, GEMM_BT_BF16, nullptr) == GEMM_BT_OK);
    REQUIRE(hipDeviceSynchronize() == hipSuccess);
    REQUIRE(hipMemcpy(c2.data(), dC, c2.size() * 2, hipMemcpyDeviceToHost) == hipSuccess);
    for (size_t i = 0; i < c2.size(); ++i) REQUIRE(c2[i] == a2[i] || (c2[i] | a2[i]) == 0x8000);  // +0 == -0

    REQUIRE(hipFree(dA) == hipSuccess && hipFree(dB) == hipSuccess && hipFree(dC) == hipSuccess);

    // all-ones again on larger shapes (every entry is K exactly in f32): an odd K (rows only 2-byte aligned, a
    // K tail of one element) on 1000 x 3000, and a long-K product through the split plan, first with a
    // workspace of the reported size, then through the library's own scratch
    auto ones = [](int64_t Mo, int64_t No, int64_t Ko, int mode) -> int {
        std::vector<uint16_t> ha((size_t)(Mo > No ? Mo : No) * Ko, bf16_of(1));
        std::vector<float> hc((size_t)Mo * No, -1.0f);
        void *a, *b, *c, *ws = nullptr;
        REQUIRE(hipMalloc(&a, (size_t)Mo * Ko * 2) == hipSuccess);
        REQUIRE(hipMalloc(&b, (size_t)No * Ko * 2) == hipSuccess);
        REQUIRE(hipMalloc(&c, hc.size() * 4) == hipSuccess);
        REQUIRE(hipMemcpy(a, ha.data(), (size_t)Mo * Ko * 2, hipMemcpyHostToDevice) == hipSuccess);
        REQUIRE(hipMemcpy(b, ha.data(), (size_t)No * Ko * 2, hipMemcpyHostToDevice) == hipSuccess);
        size_t need = 0;
        REQUIRE(gemm_bt_workspace_size(Mo, No, Ko, GEMM_BT_BF16, GEMM_BT_F32, &need) == GEMM_BT_OK);
        if (mode == 0) {
            REQUIRE(gemm_bt(a, b, c, Mo, No, Ko, GEMM_BT_BF16, GEMM_BT_F32, nullptr) == GEMM_BT_OK);
        } else if (mode == 1) {
            REQUIRE(need > 0);
            REQUIRE(hipMalloc(&ws, need) == hipSuccess);
            REQUIRE(hipMemset(ws, 0, need) == hipSuccess);
            REQUIRE(gemm_bt_ws(a, b, c, Mo, No, Ko, GEMM_BT_BF16, GEMM_BT_F32, ws, need - 16, nullptr) ==
                    GEMM_BT_ERR_INVALID_VALUE);
            REQUIRE(gemm_bt_ws(a, b, c, Mo, No, Ko, GEMM_BT_BF16, GEMM_BT_F32, ws, need, nullptr) == GEMM_BT_OK);
        } else {
            REQUIRE(gemm_bt_noalloc(a, b, c, Mo, No, Ko, GEMM_BT_BF16, GEMM_BT_F32, nullptr) == GEMM_BT_OK);
        }
        REQUIRE(hipDeviceSynchronize() == hipSuccess);
        REQUIRE(hipMemcpy(hc.data(), c, hc.size() * 4, hipMemcpyDeviceToHost) == hipSuccess);
        for (size_t i = 0; i < hc.size(); ++i) REQUIRE(hc[i] == (float)Ko);
        REQUIRE(hipFree(a) == hipSuccess && hipFree(b) == hipSuccess && hipFree(c) == hipSuccess);
        if (ws) REQUIRE(hipFree(ws) == hipSuccess);
        return 0;
    };
    REQUIRE(ones(1000, 3000, 2049, 0) == 0);
    REQUIRE(ones(1024, 1024, 16384, 1) == 0);
    REQUIRE(ones(1024, 1024, 16384, 2) == 0);
    std::printf("c_abi_check ok\n");
    return 0;
}
