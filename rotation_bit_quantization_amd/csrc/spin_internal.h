// Host-side launchers behind the libspin C ABI.  abi.cpp validates every
// argument before calling these; the launchers only pick a kernel and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spin {

// Hadamard order n = 2^log2p * (has12 ? 12 : 1).
struct HadOrder {
    int n;
    int log2p;
    bool has12;
};

// bits = 4: packed nibbles [M][K/2]; bits = 8: one signed byte per code [M][K].
hipError_t launch_fwht_quant(const void* X, bool x_f16, int M, int K, HadOrder h, int bits,
                             uint8_t* Xq, float* x_scale, float* X_rot, hipStream_t s);

hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, hipStream_t s);

hipError_t launch_kv_quant(const void* X, bool x_f16, int T, int H, bool rotate, int bits,
                           uint8_t* codes, uint16_t* scale, float* X_rot, hipStream_t s);

// Int8 activation codes [M][K] against packed INT4 weights [N][K/2]; K % 128 == 0.
hipError_t launch_w4a8_gemm(const int8_t* Xq8, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, hipStream_t s);

hipError_t launch_fold_rotation(const float* W, int K, int N, const float* R, int r_block,
                                HadOrder h, float* W_rot, uint8_t* Wq, float* w_scale,
                                hipStream_t s);

}  // namespace spin
