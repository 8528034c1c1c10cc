// Host-side launchers behind the libspin C ABI.  abi.cpp validates every
// argument before calling these; the launchers only pick a kernel and launch.
#pragma once

#include <hip/hip_fp16.h>
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

// kernel: 0 the automatic choice, 1 the int8 kernels, 2 the FP6 kernel
// (abi.cpp has checked that the FP6 kernel takes K).
hipError_t launch_w4a4_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, int kernel, hipStream_t s);

hipError_t launch_kv_quant(const void* X, bool x_f16, int T, int H, bool rotate, int bits,
                           uint8_t* codes, uint16_t* scale, float* X_rot, hipStream_t s);

// Q (optional, rotate only), K (rotate + quantize) and V (quantize) in one launch.
hipError_t launch_kv_qkv(const void* Q, const void* K, const void* V, bool x_f16, int T, int Hq, int Hkv,
                         int bits, float* Q_rot, uint8_t* K_codes, uint16_t* K_scale, float* K_rot,
                         uint8_t* V_codes, uint16_t* V_scale, hipStream_t s);

// The FP6 matrix-core path of launch_w4a4_gemm (exact for K <= kGemmFp6MaxK).
constexpr int kGemmFp6MaxK = 65536;
bool w4a4_gemm_fp6_applies(int M, int N, int K);
int w4a4_gemm_fp6_split_slices(int M, int N, int K, bool forced);
hipError_t launch_w4a4_gemm_fp6_split(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                                      const float* w_scale, int M, int N, int K, int slices, float* Y,
                                      int32_t* acc_out, hipStream_t s);
hipError_t launch_codes_f6(const uint8_t* Wq, int N, int K, uint8_t* Wf6, int32_t* w_sum, hipStream_t s);
hipError_t launch_w4a4_gemm_f6f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale,
                                 const uint8_t* Wf6, const int32_t* w_sum, const float* w_scale, int M, int N, int K,
                                 float* Y, int32_t* acc_out, hipStream_t s);
hipError_t launch_w4a4_gemm_fp6(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq,
                                const float* w_scale, int M, int N, int K, float* Y,
                                int32_t* acc_out, hipStream_t s);

// Int8 activation codes [M][K] against packed INT4 weights [N][K/2]; K % 128 == 0.
hipError_t launch_w4a8_gemm(const int8_t* Xq8, const float* x_scale, const uint8_t* Wq,
                            const float* w_scale, int M, int N, int K, float* Y,
                            int32_t* acc_out, hipStream_t s);

// fwht_quant (fp16, K = had_n = 12288, INT4) then the FP6 GEMM, one cooperative launch.
hipError_t launch_fwht_quant_gemm(const __half* X, int M, int K, const uint8_t* Wq, const float* w_scale, int N,
                                  uint8_t* Xq, float* x_scale, float* Y, int32_t* acc_out, uint32_t* workspace,
                                  hipStream_t s);

// Device address of the current device's library-owned flags for the fused
// kernel (SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS words, zero between calls),
// looked up once per device.
hipError_t fwht_quant_gemm_scratch(uint32_t** out);

// fp16 rows of 12288, H_12 (x) H_1024, INT4 codes in the FP6 operand layout + row code sums.
hipError_t launch_fwht_quant_f6(const __half* X, int M, uint8_t* Xf6, int32_t* x_sum, float* x_scale,
                                hipStream_t s);
// had_n = 1: fp16 / fp32 rows of K (K % 128 == 0, K <= SPIN_FWHT_F6_QUANT_MAX_K), per-token INT4 codes in
// the FP6 operand layout + row code sums.
hipError_t launch_quant_rows_f6(const void* X, bool x_f16, int M, int K, uint8_t* Xf6, int32_t* x_sum,
                                float* x_scale, hipStream_t s);
// The FP6 GEMM on activation codes in that layout.
hipError_t launch_w4a4_gemm_f6(const uint8_t* Xf6, const int32_t* x_sum, const float* x_scale, const uint8_t* Wq,
                               const float* w_scale, int M, int N, int K, float* Y, int32_t* acc_out,
                               hipStream_t s);

// Compute units of the current device, queried once per device and cached
// (0 if the runtime cannot tell); safe to call from several threads.
int device_cu_count();

hipError_t launch_fold_rotation(const float* W, int K, int N, const float* R, int r_block,
                                HadOrder h, float* W_rot, uint8_t* Wq, float* w_scale,
                                hipStream_t s);

}  // namespace spin
