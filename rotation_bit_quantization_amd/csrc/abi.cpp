// The libspin C ABI: host-side argument validation, then one launcher call.
// Every check happens before anything is enqueued, so a rejected call writes
// no output (declarations and contracts in include/libspin.h).
#include "libspin.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "spin_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Parses a Hadamard order: 1, 2^k (1 <= k <= 14) or 12 * 2^k (0 <= k <= 10).
bool parse_had(int n, spin::HadOrder* h) {
    if (n == 1) {
        *h = {1, 0, false};
        return true;
    }
    if (n >= 2 && n <= (1 << 14) && (n & (n - 1)) == 0) {
        *h = {n, __builtin_ctz(static_cast<unsigned>(n)), false};
        return true;
    }
    if (n >= 12 && n % 12 == 0) {
        const int m = n / 12;
        if ((m & (m - 1)) == 0 && m <= (1 << 10)) {
            *h = {n, __builtin_ctz(static_cast<unsigned>(m)), true};
            return true;
        }
    }
    return false;
}

spin_status from_hip(hipError_t e) { return e == hipSuccess ? SPIN_OK : SPIN_ERR_HIP; }

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];   // 0: not queried yet

// Shared by the 4-bit and 8-bit entry points; `bits` picks the code width.
spin_status fwht_quant_impl(const void* X, spin_dtype x_dtype, int M, int K, int had_n, int bits,
                            uint8_t* Xq, float* x_scale, float* X_rot, void* stream) {
    if (!X || !Xq || !x_scale) return SPIN_ERR_NULL;
    if (x_dtype != SPIN_F32 && x_dtype != SPIN_F16) return SPIN_ERR_UNSUPPORTED;
    spin::HadOrder h;
    if (!parse_had(had_n, &h)) return SPIN_ERR_UNSUPPORTED;
    if (M < 0 || M > SPIN_FWHT_MAX_M || K <= 0 || K > SPIN_FWHT_MAX_K || K % 32 != 0 || K % had_n != 0)
        return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(X) || !aligned16(Xq) || !aligned16(x_scale) || (X_rot && !aligned16(X_rot)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0) return SPIN_OK;
    return from_hip(spin::launch_fwht_quant(X, x_dtype == SPIN_F16, M, K, h, bits, Xq, x_scale, X_rot,
                                            static_cast<hipStream_t>(stream)));
}

spin_status kv_quant_impl(const void* X, spin_dtype x_dtype, int T, int H, int D, int rotate, int bits,
                          uint8_t* codes, uint16_t* scale, float* X_rot, void* stream) {
    if (!X) return SPIN_ERR_NULL;
    if ((codes == nullptr) != (scale == nullptr)) return SPIN_ERR_NULL;
    if (!codes && !X_rot) return SPIN_ERR_NULL;
    if (x_dtype != SPIN_F32 && x_dtype != SPIN_F16) return SPIN_ERR_UNSUPPORTED;
    if (rotate != 0 && rotate != 1) return SPIN_ERR_UNSUPPORTED;
    if (T < 0 || H < 0 || D != 128) return SPIN_ERR_BAD_SHAPE;
    if (static_cast<long long>(T) * H > SPIN_KV_MAX_VECTORS) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(X) || (codes && !aligned16(codes)) || (scale && !aligned16(scale)) ||
        (X_rot && !aligned16(X_rot)))
        return SPIN_ERR_MISALIGNED;
    if (T == 0 || H == 0) return SPIN_OK;
    return from_hip(spin::launch_kv_quant(X, x_dtype == SPIN_F16, T, H, rotate == 1, bits, codes, scale,
                                          X_rot, static_cast<hipStream_t>(stream)));
}

// spin_fwht_quant_gemm with the caller's workspace, or (workspace == NULL)
// with the library's per-device flags, looked up only once the arguments
// are valid and there is a product to compute.
spin_status fwht_quant_gemm_impl(const void* X, spin_dtype x_dtype, int M, int K, int had_n, const uint8_t* Wq,
                                 const float* w_scale, int N, uint8_t* Xq, float* x_scale, float* Y,
                                 int32_t* acc_out, uint32_t* workspace, void* stream) {
    if (!X || !Wq || !w_scale || !Xq || !x_scale || !Y) return SPIN_ERR_NULL;
    if (x_dtype != SPIN_F16 || had_n != 12288) return SPIN_ERR_UNSUPPORTED;
    if (K != 12288 || M < 0 || M > SPIN_FWHT_MAX_M || N < 0) return SPIN_ERR_BAD_SHAPE;
    const long long tiles = (static_cast<long long>(M) + 255) / 256 * ((static_cast<long long>(N) + 255) / 256);
    if (tiles > 0x7FFFFFFFLL) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(w_scale) || !aligned16(Xq) || !aligned16(x_scale) ||
        !aligned16(Y) || (acc_out && !aligned16(acc_out)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0) return SPIN_OK;
    if (N == 0)   // no product: the codes alone
        return from_hip(spin::launch_fwht_quant(X, true, M, K, spin::HadOrder{12288, 10, true}, 4, Xq, x_scale,
                                                nullptr, static_cast<hipStream_t>(stream)));
    if (!workspace && spin::fwht_quant_gemm_scratch(&workspace) != hipSuccess) return SPIN_ERR_HIP;
    return from_hip(spin::launch_fwht_quant_gemm(static_cast<const __half*>(X), M, K, Wq, w_scale, N, Xq, x_scale,
                                                 Y, acc_out, workspace, static_cast<hipStream_t>(stream)));
}

}  // namespace

int spin::device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev >= kMaxDevices) {
        int cus = 0;
        return hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? cus : 0;
    }
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    g_cu_count[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

extern "C" {

const char* spin_status_string(spin_status s) {
    switch (s) {
        case SPIN_OK: return "SPIN_OK";
        case SPIN_ERR_NULL: return "SPIN_ERR_NULL: a required pointer is NULL";
        case SPIN_ERR_BAD_SHAPE: return "SPIN_ERR_BAD_SHAPE: a size is out of range or not a required multiple";
        case SPIN_ERR_MISALIGNED: return "SPIN_ERR_MISALIGNED: a tensor pointer is not 16-byte aligned";
        case SPIN_ERR_UNSUPPORTED: return "SPIN_ERR_UNSUPPORTED: unsupported Hadamard order, dtype or flag";
        case SPIN_ERR_HIP: return "SPIN_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown spin_status";
}

int spin_version(void) { return 100; }

spin_status spin_fwht_quant(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                            uint8_t* Xq, float* x_scale, float* X_rot, void* stream) {
    return fwht_quant_impl(X, x_dtype, M, K, had_n, 4, Xq, x_scale, X_rot, stream);
}

spin_status spin_fwht_quant8(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                             int8_t* Xq8, float* x_scale, float* X_rot, void* stream) {
    return fwht_quant_impl(X, x_dtype, M, K, had_n, 8, reinterpret_cast<uint8_t*>(Xq8), x_scale, X_rot,
                           stream);
}

spin_status spin_w4a4_gemm_ex(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                              const float* w_scale, int M, int N, int K, float* Y,
                              int32_t* acc_out, int kernel, void* stream) {
    if (!Xq || !x_scale || !Wq || !w_scale || !Y) return SPIN_ERR_NULL;
    if (kernel != SPIN_GEMM_AUTO && kernel != SPIN_GEMM_INT8 && kernel != SPIN_GEMM_FP6 &&
        kernel != SPIN_GEMM_FP6_SPLITK)
        return SPIN_ERR_UNSUPPORTED;
    if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || K > SPIN_GEMM_MAX_K) return SPIN_ERR_BAD_SHAPE;
    if ((kernel == SPIN_GEMM_FP6 || kernel == SPIN_GEMM_FP6_SPLITK) &&
        (K % 128 != 0 || K < SPIN_GEMM_FP6_MIN_K || K > SPIN_GEMM_FP6_MAX_K))
        return SPIN_ERR_BAD_SHAPE;
    const long long tiles = (static_cast<long long>(M) + 127) / 128 * ((static_cast<long long>(N) + 127) / 128);
    if (tiles > 0x7FFFFFFFLL) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(Wq) || !aligned16(w_scale) ||
        !aligned16(Y) || (acc_out && !aligned16(acc_out)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0 || N == 0) return SPIN_OK;
    return from_hip(spin::launch_w4a4_gemm(Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out, kernel,
                                           static_cast<hipStream_t>(stream)));
}

spin_status spin_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                           const float* w_scale, int M, int N, int K, float* Y,
                           int32_t* acc_out, void* stream) {
    return spin_w4a4_gemm_ex(Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out, SPIN_GEMM_AUTO, stream);
}

spin_status spin_fwht_quant_gemm(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                                 const uint8_t* Wq, const float* w_scale, int N, uint8_t* Xq,
                                 float* x_scale, float* Y, int32_t* acc_out, uint32_t* workspace,
                                 void* stream) {
    if (!workspace) return SPIN_ERR_NULL;
    if (!aligned16(workspace)) return SPIN_ERR_MISALIGNED;
    return fwht_quant_gemm_impl(X, x_dtype, M, K, had_n, Wq, w_scale, N, Xq, x_scale, Y, acc_out, workspace,
                                stream);
}

spin_status spin_fwht_quant_gemm_noalloc(const void* X, spin_dtype x_dtype, int M, int K, int had_n,
                                         const uint8_t* Wq, const float* w_scale, int N, uint8_t* Xq,
                                         float* x_scale, float* Y, int32_t* acc_out, void* stream) {
    return fwht_quant_gemm_impl(X, x_dtype, M, K, had_n, Wq, w_scale, N, Xq, x_scale, Y, acc_out, nullptr,
                                stream);
}

spin_status spin_fwht_quant_f6(const void* X, spin_dtype x_dtype, int M, int K, int had_n, uint8_t* Xf6,
                               int32_t* x_sum, float* x_scale, void* stream) {
    if (!X || !Xf6 || !x_sum || !x_scale) return SPIN_ERR_NULL;
    if (had_n == 12288) {
        if (x_dtype != SPIN_F16) return SPIN_ERR_UNSUPPORTED;
        if (K != 12288) return SPIN_ERR_BAD_SHAPE;
    } else if (had_n == 1) {
        if (x_dtype != SPIN_F16 && x_dtype != SPIN_F32) return SPIN_ERR_UNSUPPORTED;
        if (K % 128 != 0 || K < SPIN_GEMM_FP6_MIN_K || K > SPIN_FWHT_F6_QUANT_MAX_K) return SPIN_ERR_BAD_SHAPE;
    } else {
        return SPIN_ERR_UNSUPPORTED;
    }
    if (M < 0 || M > SPIN_FWHT_MAX_M) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(X) || !aligned16(Xf6) || !aligned16(x_sum) || !aligned16(x_scale)) return SPIN_ERR_MISALIGNED;
    if (M == 0) return SPIN_OK;
    if (had_n == 1)
        return from_hip(spin::launch_quant_rows_f6(X, x_dtype == SPIN_F16, M, K, Xf6, x_sum, x_scale,
                                                   static_cast<hipStream_t>(stream)));
    return from_hip(spin::launch_fwht_quant_f6(static_cast<const __half*>(X), M, Xf6, x_sum, x_scale,
                                               static_cast<hipStream_t>(stream)));
}

spin_status spin_w4a4_gemm_f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale,
                              const uint8_t* Wq, const float* w_scale, int M, int N, int K, float* Y,
                              int32_t* acc_out, void* stream) {
    if (!Xf6 || !x_sum || !x_scale || !Wq || !w_scale || !Y) return SPIN_ERR_NULL;
    if (M < 0 || N < 0 || K % 128 != 0 || K < SPIN_GEMM_FP6_MIN_K || K > SPIN_GEMM_FP6_MAX_K)
        return SPIN_ERR_BAD_SHAPE;
    const long long tiles = (static_cast<long long>(M) + 255) / 256 * ((static_cast<long long>(N) + 255) / 256);
    if (tiles > 0x7FFFFFFFLL) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(Xf6) || !aligned16(x_sum) || !aligned16(x_scale) || !aligned16(Wq) || !aligned16(w_scale) ||
        !aligned16(Y) || (acc_out && !aligned16(acc_out)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0 || N == 0) return SPIN_OK;
    return from_hip(spin::launch_w4a4_gemm_f6(Xf6, x_sum, x_scale, Wq, w_scale, M, N, K, Y, acc_out,
                                              static_cast<hipStream_t>(stream)));
}

spin_status spin_codes_f6(const uint8_t* Wq, int N, int K, uint8_t* Wf6, int32_t* w_sum, void* stream) {
    if (!Wq || !Wf6 || !w_sum) return SPIN_ERR_NULL;
    if (N < 0 || K <= 0 || K % 64 != 0 || K > SPIN_GEMM_MAX_K) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(Wq) || !aligned16(Wf6) || !aligned16(w_sum)) return SPIN_ERR_MISALIGNED;
    if (N == 0) return SPIN_OK;
    return from_hip(spin::launch_codes_f6(Wq, N, K, Wf6, w_sum, static_cast<hipStream_t>(stream)));
}

spin_status spin_w4a4_gemm_f6f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale,
                                const uint8_t* Wf6, const int32_t* w_sum, const float* w_scale, int M, int N,
                                int K, float* Y, int32_t* acc_out, void* stream) {
    if (!Xf6 || !x_sum || !x_scale || !Wf6 || !w_sum || !w_scale || !Y) return SPIN_ERR_NULL;
    if (M < 0 || N < 0 || K % 128 != 0 || K < SPIN_GEMM_FP6_MIN_K || K > SPIN_GEMM_FP6_MAX_K)
        return SPIN_ERR_BAD_SHAPE;
    const long long tiles = (static_cast<long long>(M) + 255) / 256 * ((static_cast<long long>(N) + 255) / 256);
    if (tiles > 0x7FFFFFFFLL) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(Xf6) || !aligned16(x_sum) || !aligned16(x_scale) || !aligned16(Wf6) || !aligned16(w_sum) ||
        !aligned16(w_scale) || !aligned16(Y) || (acc_out && !aligned16(acc_out)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0 || N == 0) return SPIN_OK;
    return from_hip(spin::launch_w4a4_gemm_f6f6(Xf6, x_sum, x_scale, Wf6, w_sum, w_scale, M, N, K, Y, acc_out,
                                                static_cast<hipStream_t>(stream)));
}

spin_status spin_kv_quant(const void* X, spin_dtype x_dtype, int T, int H, int D, int rotate,
                          uint8_t* codes, uint16_t* scale, float* X_rot, void* stream) {
    return kv_quant_impl(X, x_dtype, T, H, D, rotate, 4, codes, scale, X_rot, stream);
}

spin_status spin_kv_quant8(const void* X, spin_dtype x_dtype, int T, int H, int D, int rotate,
                           int8_t* codes, uint16_t* scale, float* X_rot, void* stream) {
    return kv_quant_impl(X, x_dtype, T, H, D, rotate, 8, reinterpret_cast<uint8_t*>(codes), scale, X_rot,
                         stream);
}

spin_status spin_kv_qkv(const void* Q, const void* K, const void* V, spin_dtype x_dtype, int T, int Hq,
                        int Hkv, int D, int bits, float* Q_rot, uint8_t* K_codes, uint16_t* K_scale,
                        float* K_rot, uint8_t* V_codes, uint16_t* V_scale, void* stream) {
    if (!K || !V || !K_codes || !K_scale || !V_codes || !V_scale) return SPIN_ERR_NULL;
    if ((Q == nullptr) != (Q_rot == nullptr)) return SPIN_ERR_NULL;
    if (x_dtype != SPIN_F32 && x_dtype != SPIN_F16) return SPIN_ERR_UNSUPPORTED;
    if (bits != 4 && bits != 8) return SPIN_ERR_UNSUPPORTED;
    if (T < 0 || Hkv < 0 || (Q && Hq < 0) || D != 128) return SPIN_ERR_BAD_SHAPE;
    {   // the one launch's workgroups: K and V 32 vectors each, then Q (as launch_kv_qkv counts them)
        const long long gkv = static_cast<long long>(T) * Hkv, gq = Q ? static_cast<long long>(T) * Hq : 0;
        if (2 * ((gkv + 31) / 32) + (gq + 31) / 32 > (1LL << 24) - 1) return SPIN_ERR_BAD_SHAPE;
    }
    if ((Q && (!aligned16(Q) || !aligned16(Q_rot))) || !aligned16(K) || !aligned16(V) || !aligned16(K_codes) ||
        !aligned16(K_scale) || (K_rot && !aligned16(K_rot)) || !aligned16(V_codes) || !aligned16(V_scale))
        return SPIN_ERR_MISALIGNED;
    if (T == 0 || (Hkv == 0 && (!Q || Hq == 0))) return SPIN_OK;
    return from_hip(spin::launch_kv_qkv(Q, K, V, x_dtype == SPIN_F16, T, Q ? Hq : 0, Hkv, bits, Q_rot, K_codes,
                                        K_scale, K_rot, V_codes, V_scale, static_cast<hipStream_t>(stream)));
}

spin_status spin_w4a8_gemm(const int8_t* Xq8, const float* x_scale, const uint8_t* Wq,
                           const float* w_scale, int M, int N, int K, float* Y,
                           int32_t* acc_out, void* stream) {
    if (!Xq8 || !x_scale || !Wq || !w_scale || !Y) return SPIN_ERR_NULL;
    if (M < 0 || N < 0 || K <= 0 || K % 128 != 0 || K > SPIN_GEMM8_MAX_K) return SPIN_ERR_BAD_SHAPE;
    const long long tiles = (static_cast<long long>(M) + 255) / 256 * ((static_cast<long long>(N) + 255) / 256);
    if (tiles > 0x7FFFFFFFLL) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(Xq8) || !aligned16(x_scale) || !aligned16(Wq) || !aligned16(w_scale) ||
        !aligned16(Y) || (acc_out && !aligned16(acc_out)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0 || N == 0) return SPIN_OK;
    return from_hip(spin::launch_w4a8_gemm(Xq8, x_scale, Wq, w_scale, M, N, K, Y, acc_out,
                                           static_cast<hipStream_t>(stream)));
}

spin_status spin_fold_rotation(const float* W, int K, int N, const float* R, int r_block,
                               float* W_rot, uint8_t* Wq, float* w_scale, void* stream) {
    if (!W || !W_rot || !Wq || !w_scale) return SPIN_ERR_NULL;
    spin::HadOrder h = {1, 0, false};
    if (r_block < 1) return SPIN_ERR_BAD_SHAPE;
    if (!R && !parse_had(r_block, &h)) return SPIN_ERR_UNSUPPORTED;
    if (K <= 0 || N < 0 || K % 64 != 0 || K % r_block != 0) return SPIN_ERR_BAD_SHAPE;
    if (static_cast<long long>(K) * N > (1LL << 38)) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(W) || (R && !aligned16(R)) || !aligned16(W_rot) || !aligned16(Wq) ||
        !aligned16(w_scale))
        return SPIN_ERR_MISALIGNED;
    if (N == 0) return SPIN_OK;
    return from_hip(spin::launch_fold_rotation(W, K, N, R, r_block, h, W_rot, Wq, w_scale,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
