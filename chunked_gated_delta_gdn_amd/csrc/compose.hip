// Exclusive prefix scan over segment transition pairs (MaxText PR "Add
// context parallelism to the Gated Delta Net", section "Implementation",
// phase 2):  h_in[0] = h0,  h_in[r+1] = M[r] h_in[r] + U[r],
// h_final = M[R-1] h_in[R-1] + U[R-1].
// Batch mode walks the R segments of a (sequence, head) with state rows
// [R, N, H]; packed mode walks the pieces of one sequence (rows [P, H]) from
// its piece `first` on.  With `reverse` the steps run last to first (the
// backward pass composes its reverse scan so, with M holding the transposed
// maps): h_in of the last step is h0, and each earlier one is M h + U of the
// step after it.
//
// The NS strips of one (sequence, head) all read the same M rows, so they are
// placed on one XCD (workgroups go to the 8 XCDs in turn by index, and each
// XCD has its own L2): M is then fetched from HBM about once per pair.
//
// The columns of the state are independent under h <- M h + U, so one
// workgroup owns a 16-column strip of one (sequence, head) state and walks
// the R segments in order; everything stays fp32 (the state is fp32).
//  * K = V = 128: fp32 matrix-core products (v_mfma_f32_16x16x4_f32).  Each
//    of the 4 waves owns 32 rows of the new strip: its rows of M[r] go
//    straight from memory into A operands (16-byte runs, issued before the
//    products), the running strip sits transposed in LDS and is read as B
//    operands, and U[r] seeds the accumulators.  One barrier per segment.
//  * other shapes: fp32 FMAs with M[r] staged in LDS.
// Work is R * 2*K*K*V flops per head, negligible next to the scan.
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kStrip = 16;

// Steps r0 .. r1-1 of the (sequence, head) pair nh, and the state row of step r.
struct Steps {
    int r0, r1;
};
__device__ __forceinline__ Steps compose_steps(const ComposeArgs &a, int64_t nh) {
    if (!a.packed) return {0, a.R};
    const int n = (int)(nh / a.H);
    return {a.seq_first[n] + a.first, a.seq_first[n + 1]};
}
__device__ __forceinline__ int64_t compose_row(const ComposeArgs &a, int r, int64_t nh) {
    return a.packed ? (int64_t)r * a.H + nh % a.H : (int64_t)r * a.N * a.H + nh;
}
// step i (0 .. r1 - r0 - 1) of the walk
__device__ __forceinline__ int compose_step(const ComposeArgs &a, const Steps &st, int i) {
    return a.reverse ? st.r1 - 1 - i : st.r0 + i;
}
// (sequence, head) pair and strip of this workgroup: the strips of a pair
// share an XCD (see above); pairs past N * H (grid padding) get nh = -1
constexpr int kXcds = 8;
template <int NS>
__device__ __forceinline__ void compose_unit(const ComposeArgs &a, int64_t &nh, int &strip) {
    const int64_t b = blockIdx.x, idx = b / kXcds;
    strip = (int)(idx % NS);
    nh = (idx / NS) * kXcds + b % kXcds;
    if (nh >= (int64_t)a.N * a.H) nh = -1;
}

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
    int64_t nh;   // (n, h) flattened
    int strip;
    compose_unit<NS>(a, nh, strip);
    if (nh < 0) return;
    const Steps st = compose_steps(a, nh);
    const int j = tid % kStrip, rg = tid / kStrip;
    const int c0 = strip * kStrip;

    for (int e = tid; e < K * kStrip; e += kThreads) {
        const int i = e / kStrip, jj = e % kStrip;
        sh[e] = a.h0 ? a.h0[(nh * K + i) * V + c0 + jj] : 0.f;
    }
    __syncthreads();

    for (int i0 = 0; i0 < st.r1 - st.r0; ++i0) {
        const int r = compose_step(a, st, i0);
        const int64_t slot = compose_row(a, r, nh);
        for (int e = tid; e < K * kStrip; e += kThreads) {
            const int i = e / kStrip, jj = e % kStrip;
            a.h_in[(slot * K + i) * V + c0 + jj] = sh[e];
        }
        if (i0 == st.r1 - st.r0 - 1 && !a.h_final) break;
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

// K = V = 128 on the matrix cores.  In a 16x16x4 fp32 product lane (i, g)
// (i = lane % 16, g = lane / 16) supplies A[i][g] and B[g][i] and receives
// D[4g + e][i].  Step s = 4q + e of the reduction gives lane group g the
// index k = 4 (4q + g) + e, so a lane's A operands for q are one 16-byte run
// of its row of M, and its B operands one 16-byte run of the transposed strip.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kThreads) void compose_mfma_kernel(ComposeArgs a) {
    constexpr int K = 128, V = 128, NS = V / kStrip, LD = K + 4;
    __shared__ __attribute__((aligned(16))) float hT[2][kStrip * LD];   // [column][row], two copies

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    int64_t nh;
    int strip;
    compose_unit<NS>(a, nh, strip);
    if (nh < 0) return;
    const Steps st = compose_steps(a, nh);
    const int c0 = strip * kStrip;

    for (int e = tid; e < K * kStrip; e += kThreads) {
        const int i = e / kStrip, jj = e % kStrip;
        hT[0][jj * LD + i] = a.h0 ? a.h0[(nh * K + i) * V + c0 + jj] : 0.f;
    }
    __syncthreads();
    int cur = 0;
    for (int i0 = 0; i0 < st.r1 - st.r0; ++i0) {
        const int r = compose_step(a, st, i0);
        const int64_t slot = compose_row(a, r, nh);
        for (int e = tid; e < K * kStrip; e += kThreads) {
            const int i = e / kStrip, jj = e % kStrip;
            a.h_in[(slot * K + i) * V + c0 + jj] = hT[cur][jj * LD + i];
        }
        if (i0 == st.r1 - st.r0 - 1 && !a.h_final) break;
        const float *Mr = a.M + slot * K * K;
        f32x4 ma[2][8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int q = 0; q < 8; ++q)
                ma[rb][q] = *reinterpret_cast<const f32x4 *>(&Mr[(32 * w + 16 * rb + li) * K + 4 * (4 * q + lg)]);
        f32x4 acc[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rb][e] = a.U[(slot * K + 32 * w + 16 * rb + 4 * lg + e) * V + c0 + li];
        const float *hc = hT[cur];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 hb = *reinterpret_cast<const f32x4 *>(&hc[li * LD + 4 * (4 * q + lg)]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    acc[rb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ma[rb][q][e], hb[e], acc[rb], 0, 0, 0);
        }
        // lane (j, g) holds rows 32w + 16rb + 4g + e of column j
        float *hn = hT[cur ^ 1];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) *reinterpret_cast<f32x4 *>(&hn[li * LD + 32 * w + 16 * rb + 4 * lg]) = acc[rb];
        __syncthreads();
        cur ^= 1;
    }
    if (a.h_final) {
        for (int e = tid; e < K * kStrip; e += kThreads) {
            const int i = e / kStrip, jj = e % kStrip;
            a.h_final[(nh * K + i) * V + c0 + jj] = hT[cur][jj * LD + i];
        }
    }
}

// workgroups: N * H pairs rounded up to whole XCD groups, times the strips
int64_t compose_grid(const ComposeArgs &a, int V) {
    const int64_t pairs = (int64_t)a.N * a.H;
    return (pairs + kXcds - 1) / kXcds * kXcds * (V / kStrip);
}

}  // namespace

hipError_t launch_compose(int K, int V, const ComposeArgs &a, hipStream_t s) {
    const int64_t n = compose_grid(a, V);
    if (n == 0) return hipSuccess;
    if (K == 32 && V == 32)
        hipLaunchKernelGGL((compose_kernel<32, 32>), dim3((unsigned)n), dim3(kThreads), 0, s, a);
    else if (K == 128 && V == 128)
        hipLaunchKernelGGL(compose_mfma_kernel, dim3((unsigned)n), dim3(kThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
