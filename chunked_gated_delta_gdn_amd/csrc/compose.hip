// Exclusive prefix scan over segment transition pairs (MaxText PR "Add
// context parallelism to the Gated Delta Net", section "Implementation",
// phase 2):  h_in[0] = h0,  h_in[r+1] = M[r] h_in[r] + U[r],
// h_final = M[R-1] h_in[R-1] + U[R-1].
//
// The columns of the state are independent under h <- M h + U, so one
// workgroup owns a 16-column strip of one (sequence, head) state and walks
// the R segments in order.  M[r] (K x K fp32) is staged whole in LDS, the
// strip of the running state too; fp32 FMAs throughout (the state is fp32).
// Work is R * 2*K*K*V flops per head, negligible next to the scan.
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kStrip = 16;

template <int K, int V>
__global__ __launch_bounds__(kThreads) void compose_kernel(ComposeArgs a) {
    constexpr int KP = K + 1;
    constexpr int NS = V / kStrip;
    constexpr int RG = kThreads / kStrip;   // row groups
    constexpr int RPT = K / RG;             // rows per thread
    static_assert(V % kStrip == 0 && K % RG == 0, "compose tiling");
    __shared__ float sM[K * KP];
    __shared__ float sh[K * kStrip];

    const int tid = threadIdx.x;
    const int strip = blockIdx.x % NS;
    const int64_t nh = blockIdx.x / NS;        // (n, h) flattened
    const int64_t NH = (int64_t)a.N * a.H;
    const int j = tid % kStrip, rg = tid / kStrip;
    const int c0 = strip * kStrip;

    for (int e = tid; e < K * kStrip; e += kThreads) {
        const int i = e / kStrip, jj = e % kStrip;
        sh[e] = a.h0 ? a.h0[(nh * K + i) * V + c0 + jj] : 0.f;
    }
    __syncthreads();

    for (int r = 0; r < a.R; ++r) {
        const int64_t slot = (int64_t)r * NH + nh;
        for (int e = tid; e < K * kStrip; e += kThreads) {
            const int i = e / kStrip, jj = e % kStrip;
            a.h_in[(slot * K + i) * V + c0 + jj] = sh[e];
        }
        if (r == a.R - 1 && !a.h_final) break;
        const float *Mr = a.M + slot * K * K;
        for (int e = tid; e < K * K; e += kThreads) sM[(e / K) * KP + e % K] = Mr[e];
        __syncthreads();
        float acc[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg * RPT + m;
            acc[m] = a.U[(slot * K + i) * V + c0 + j];
        }
        for (int l = 0; l < K; ++l) {
            const float hl = sh[l * kStrip + j];
#pragma unroll
            for (int m = 0; m < RPT; ++m) acc[m] = fmaf(sM[(rg * RPT + m) * KP + l], hl, acc[m]);
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < RPT; ++m) sh[(rg * RPT + m) * kStrip + j] = acc[m];
        __syncthreads();
    }
    if (a.h_final) {
        for (int e = tid; e < K * kStrip; e += kThreads) {
            const int i = e / kStrip, jj = e % kStrip;
            a.h_final[(nh * K + i) * V + c0 + jj] = sh[e];
        }
    }
}

template <int K, int V>
hipError_t launch_t(const ComposeArgs &a, hipStream_t s) {
    const int64_t n = (int64_t)a.N * a.H * (V / kStrip);
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((compose_kernel<K, V>), dim3((unsigned)n), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_compose(int K, int V, const ComposeArgs &a, hipStream_t s) {
    if (K == 32 && V == 32) return launch_t<32, 32>(a, s);
    if (K == 128 && V == 128) return launch_t<128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
