// The libspin C ABI: host-side argument validation, then one launcher call.
// Every check happens before anything is enqueued, so a rejected call writes
// no output (declarations and contracts in include/libspin.h).
#include "libspin.h"

#include <hip/hip_runtime.h>

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

// Shared by the 4-bit and 8-bit entry points; `bits` picks the code width.
spin_status fwht_quant_impl(const void* X, spin_dtype x_dtype, int M, int K, int had_n, int bits,
                            uint8_t* Xq, float* x_scale, float* X_rot, void* stream) {
    if (!X || !Xq || !x_scale) return SPIN_ERR_NULL;
    if (x_dtype != SPIN_F32 && x_dtype != SPIN_F16) return SPIN_ERR_UNSUPPORTED;
    spin::HadOrder h;
    if (!parse_had(had_n, &h)) return SPIN_ERR_UNSUPPORTED;
    if (M < 0 || K <= 0 || K > SPIN_FWHT_MAX_K || K % 32 != 0 || K % had_n != 0)
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
    if (static_cast<long long>(T) * H > (1LL << 34)) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(X) || (codes && !aligned16(codes)) || (scale && !aligned16(scale)) ||
        (X_rot && !aligned16(X_rot)))
        return SPIN_ERR_MISALIGNED;
    if (T == 0 || H == 0) return SPIN_OK;
    return from_hip(spin::launch_kv_quant(X, x_dtype == SPIN_F16, T, H, rotate == 1, bits, codes, scale,
                                          X_rot, static_cast<hipStream_t>(stream)));
}

}  // namespace

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

spin_status spin_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                           const float* w_scale, int M, int N, int K, float* Y,
                           int32_t* acc_out, void* stream) {
    if (!Xq || !x_scale || !Wq || !w_scale || !Y) return SPIN_ERR_NULL;
    if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || K > SPIN_GEMM_MAX_K) return SPIN_ERR_BAD_SHAPE;
    const long long tiles = (static_cast<long long>(M) + 127) / 128 * ((static_cast<long long>(N) + 127) / 128);
    if (tiles > 0x7FFFFFFFLL) return SPIN_ERR_BAD_SHAPE;
    if (!aligned16(Xq) || !aligned16(x_scale) || !aligned16(Wq) || !aligned16(w_scale) ||
        !aligned16(Y) || (acc_out && !aligned16(acc_out)))
        return SPIN_ERR_MISALIGNED;
    if (M == 0 || N == 0) return SPIN_OK;
    return from_hip(spin::launch_w4a4_gemm(Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out,
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
