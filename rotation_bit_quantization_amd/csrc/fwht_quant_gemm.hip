// spin_fwht_quant_gemm: the down projection's online R4 Hadamard and per-token
// INT4 quantizer as the prologue of its W4A4 GEMM, in one launch (page
// "SpinQuant, Reproduced", Q5: R4 runs online right before down_proj;
// abstract: W4A4).
//
// Persistent workgroups, one per compute unit (the FP6 tile's 144 KB of LDS
// leaves room for no second), launched cooperatively so that all of them are
// resident at once:
//   phase 1  workgroup b transforms and quantizes rows [b R, (b + 1) R),
//            R = ceil(M / G), one row per wave at a time (fwht12288_row, the
//            code of the one-wave fwht_quant kernel), writing codes and
//            scales to Xq / x_scale exactly as spin_fwht_quant does; then it
//            publishes its flag (release at device scope: the codes are
//            written back past this XCD's L2 before the flag is seen);
//   phase 2  workgroup b takes tiles b, b + G, ... in the XCD-aware order of
//            the FP6 GEMM; before a tile its first thread waits (acquire)
//            for the flags of the workgroups that produced the tile's 256
//            rows, then the workgroup multiplies them (fp6::gemm_tile).
// A tile can start as soon as its own rows are done, so the last rows of
// phase 1 overlap the first tiles of phase 2 and no launch separates them.
// The last workgroup to finish (a counter after the flags) clears flags and
// counter, so the workspace is zero again when the kernel ends.
// No wait depends on a workgroup that is not running (all G are resident and
// phase 1 waits for nothing), so every wait ends; it is bounded anyway, at
// about half a second of the 100 MHz clock or 2^22 polls, after which the
// tile is written as NaN (acc_out INT32_MIN) instead of computed.
//
// Measured on MI355X (4096 x 12288 fp16 -> 4096, the whole step timed by HIP
// events): 272 us as this one launch against 193-212 us as the two calls.
// Timestamps of the 100 MHz clock per workgroup place the loss: phase 1 ends
// at 31-41 us (the separate kernel takes 35-39 us for the same rows), the
// first tile starts only at 65-71 us (the device-scope release of 256
// workgroups, each writing its XCD's L2 back for the others, and the acquire
// that invalidates them), and a tile takes 180 us against 174 us alone.  The
// launch boundary this removes costs a few microseconds, and the codes'
// round trip through HBM (50 MB) about six, so even a free synchronisation
// would only bring the fused step level with the two calls.
#include "fwht12288.h"
#include "gemm_fp6_tile.h"
#include "libspin.h"
#include "spin_internal.h"

#include <atomic>

namespace spin {
namespace {

using namespace fp6;

constexpr int kFusedMaxGrid = SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS - 1;   // the counter follows the flags
constexpr unsigned long long kWaitTicks = 50000000ull;                   // 0.5 s at 100 MHz
constexpr unsigned kMaxPolls = 1u << 22;   // and a bound that needs no clock (seconds of polling)

template <bool WRITE_ACC>
__global__ __launch_bounds__(kF6Threads) void fwht_quant_gemm_kernel(
    const __half* __restrict__ X, float norm, float mone, int M, int N, int K,
    const uint8_t* __restrict__ Wq, const float* __restrict__ w_scale, uint8_t* __restrict__ Xq,
    float* __restrict__ x_scale, float* __restrict__ Y, int32_t* __restrict__ acc_out,
    unsigned* __restrict__ flags, int rows_per_wg) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[3 * kF6StageBytes];
    __shared__ int rows_ready;
    const int G = static_cast<int>(gridDim.x);
    const int b = static_cast<int>(blockIdx.x);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // phase 1: this workgroup's rows, one per wave at a time.  The row's
    // inputs pass through an empty asm every iteration: values hoisted out of
    // the loop would stay live through the row's peak register use and spill.
    const int r0 = b * rows_per_wg;
    const int r1 = min(M, r0 + rows_per_wg);
    for (int row = r0 + wave; row < r1; row += kF6Threads / 64) {
        const __half* x = X;
        uint8_t* q = Xq;
        float* s = x_scale;
        float n = norm, m = mone;
        int l = threadIdx.x & 63;
        asm volatile("" : "+s"(x), "+s"(q), "+s"(s), "+s"(n), "+s"(m), "+v"(l));
        fwht12288_row<4, false>(x, static_cast<size_t>(row), l, n, m, q, s, nullptr);
    }
    // After the barrier every wave's stores have reached this XCD's L2; one
    // release by the first thread then writes the L2 back for the other XCDs
    // (a release from every wave would write it back eight times over).
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(&flags[b], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);

    // phase 2: tiles in the order of the FP6 GEMM
    const int tiles_m = (M + kF6T - 1) / kF6T, tiles_n = (N + kF6T - 1) / kF6T;
    const int tiles = tiles_m * tiles_n;
    for (int t = b; t < tiles; t += G) {
        int tm, tn;
        tile_of(t, tiles_m, tiles_n, &tm, &tn);
        if (threadIdx.x == 0) {
            const int lo = (tm * kF6T) / rows_per_wg;
            const int hi = (min(M, tm * kF6T + kF6T) - 1) / rows_per_wg;
            const unsigned long long t0 = wall_clock64();
            int ok = 1;
            unsigned polls = 0;
            for (int p = lo; p <= hi && ok; ++p)
                while (__hip_atomic_load(&flags[p], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
                    if (wall_clock64() - t0 > kWaitTicks || ++polls > kMaxPolls) {
                        ok = 0;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            rows_ready = ok;
        }
        // The first thread's acquire loads have invalidated this CU's and
        // XCD's caches of the rows; the barrier orders every thread's reads
        // after them.  It also keeps the previous tile's epilogue reads of the
        // first stage before this tile's writes to it.
        __syncthreads();
        if (rows_ready) {
            gemm_tile<WRITE_ACC>(Xq, x_scale, Wq, w_scale, M, N, K, Y, acc_out, tm, tn, lds);
        } else {
            for (int e = threadIdx.x; e < kF6T * kF6T; e += kF6Threads) {
                const int row = tm * kF6T + e / kF6T, col = tn * kF6T + e % kF6T;
                if (row < M && col < N) {
                    Y[static_cast<size_t>(row) * N + col] = __builtin_nanf("");
                    if (WRITE_ACC) acc_out[static_cast<size_t>(row) * N + col] = INT32_MIN;
                }
            }
        }
        __syncthreads();   // every thread has read rows_ready before it is written again
    }

    // the last workgroup out clears the workspace for the next call
    if (threadIdx.x == 0) {
        const unsigned out = __hip_atomic_fetch_add(&flags[kFusedMaxGrid], 1u, __ATOMIC_ACQ_REL,
                                                    __HIP_MEMORY_SCOPE_AGENT);
        if (out == static_cast<unsigned>(G - 1)) {
            for (int p = 0; p < G; ++p) __hip_atomic_store(&flags[p], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&flags[kFusedMaxGrid], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Workgroups per compute unit the kernel can keep resident (1: its LDS),
// queried once per device and instantiation.
std::atomic<int> g_occupancy[2][64];

template <bool WRITE_ACC>
int resident_per_cu() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    std::atomic<int>* slot = dev < 64 ? &g_occupancy[WRITE_ACC][dev] : nullptr;
    if (slot) {
        const int v = slot->load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwht_quant_gemm_kernel<WRITE_ACC>, kF6Threads, 0) !=
            hipSuccess ||
        n <= 0)
        return 0;
    if (slot) slot->store(n, std::memory_order_relaxed);
    return n;
}

template <bool WRITE_ACC>
hipError_t launch_t(const __half* X, int M, int N, int K, const uint8_t* Wq, const float* w_scale, uint8_t* Xq,
                    float* x_scale, float* Y, int32_t* acc_out, unsigned* flags, hipStream_t s) {
    const int cus = device_cu_count();
    const int per_cu = resident_per_cu<WRITE_ACC>();
    if (cus <= 0 || per_cu <= 0) return hipErrorInvalidDevice;
    const int G = min(cus * per_cu, kFusedMaxGrid);
    int rows_per_wg = (M + G - 1) / G;
    float norm = static_cast<float>(1.0 / __builtin_sqrt(12288.0));
    float mone = -1.0f;
    void* args[] = {&X, &norm, &mone, &M, &N, &K, &Wq, &w_scale, &Xq, &x_scale, &Y, &acc_out, &flags, &rows_per_wg};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fwht_quant_gemm_kernel<WRITE_ACC>), dim3(G),
                                      dim3(kF6Threads), args, 0, s);
}

// The flags of spin_fwht_quant_gemm_noalloc: one array per device (each
// device holds its own copy of the module's globals until the process ends),
// zero when the module loads; every call leaves it zero again.  Host code
// never passes the array's name to a kernel: its device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint32_t scratch[SPIN_FWHT_QUANT_GEMM_WORKSPACE_WORDS];

constexpr int kScratchDevices = 64;
std::atomic<uint32_t*> g_scratch[kScratchDevices];

}  // namespace

hipError_t fwht_quant_gemm_scratch(uint32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    uint32_t* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        p = static_cast<uint32_t*>(q);
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
}

hipError_t launch_fwht_quant_gemm(const __half* X, int M, int K, const uint8_t* Wq, const float* w_scale, int N,
                                  uint8_t* Xq, float* x_scale, float* Y, int32_t* acc_out, uint32_t* workspace,
                                  hipStream_t s) {
    if (acc_out) return launch_t<true>(X, M, N, K, Wq, w_scale, Xq, x_scale, Y, acc_out, workspace, s);
    return launch_t<false>(X, M, N, K, Wq, w_scale, Xq, x_scale, Y, acc_out, workspace, s);
}

}  // namespace spin
