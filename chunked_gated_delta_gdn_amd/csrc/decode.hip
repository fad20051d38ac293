// Recurrent decode step: one new token per sequence, in place on the fp32
// state (the GDR decode kernel of "RFC(qwen35): TP Phase 2", section "Kernel
// Work", with the per-request recurrent state [H_v, K, V] f32 of section
// "Partition Contract"; the update is the token recurrence of the gated
// delta rule).
//
// Per (b, h), with alpha = exp(g), the state h [K, V] is read once and
// written once:
//   hk = h^T k, hq = h^T q            (column reductions over K, old state)
//   delta = beta (v - alpha hk)
//   h <- alpha h + k delta^T
//   o = h_new^T q = alpha hq + delta (k . q)
// so the output needs no second pass over the new state.
//
// Roofline: 2*K*V*4 bytes of state traffic per head against ~7*K*V flops, an
// HBM stream.  One workgroup per (b, h) with one thread per 16 bytes of four
// state rows (1024 threads at K = V = 128): a thread owns 4 adjacent columns
// (one 16-byte vector per row) for K/RS rows, so every load and store is a
// coalesced dwordx4, the whole state slice is in registers between the read
// and the write, and each thread has only a few loads to wait for.  State
// accesses are non-temporal: every byte is touched once per step and the
// state of a batch is far larger than the caches, so the stream is kept from
// displacing other lines (on MI355X this took the 512 MiB step from 64% to
// 72% of HBM bandwidth, above a plain device copy).
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float4 *p) {
    const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_nt(float4 v, float4 *p) {
    const f32x4v x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4v *>(p));
}

template <int K, int V>
constexpr int threads_for() { return K * V / 4 >= 1024 ? 1024 : K * V / 4; }

template <typename T, int K, int V>
__global__ __launch_bounds__((threads_for<K, V>())) void decode_step_kernel(DecodeArgs a) {
    constexpr int kThreads = threads_for<K, V>();
    constexpr int CG = V / 4;            // column groups of 4
    constexpr int RS = kThreads / CG;    // row sets
    constexpr int RPT = K / RS;          // rows per thread
    static_assert(V % 4 == 0 && kThreads % CG == 0 && K % RS == 0, "decode tiling");

    __shared__ float sk[K], sq[K];
    __shared__ float red_k[RS][V], red_q[RS][V];
    __shared__ float red_kq[RS];

    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.x;
    const int cg = tid % CG, rs = tid / CG;

    // q, k of the key head this value head reads (grouped order)
    const int64_t bhk = (bh / a.H) * a.Hk + (bh % a.H) / (a.H / a.Hk);
    for (int i = tid; i < K; i += kThreads) {
        sk[i] = Elem<T>::load(a.k, bhk * K + i);
        sq[i] = Elem<T>::load(a.q, bhk * K + i);
    }
    const float alpha = expf(a.g[bh]);
    const float beta = a.beta[bh];

    float4 *st = reinterpret_cast<float4 *>(a.state + bh * (int64_t)K * V);
    float4 hv[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) hv[m] = load_nt(&st[(rs + RS * m) * CG + cg]);
    __syncthreads();

    float hk[4] = {0.f, 0.f, 0.f, 0.f}, hq[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rs + RS * m;
        const float ki = sk[i], qi = sq[i];
        hk[0] = fmaf(hv[m].x, ki, hk[0]);
        hk[1] = fmaf(hv[m].y, ki, hk[1]);
        hk[2] = fmaf(hv[m].z, ki, hk[2]);
        hk[3] = fmaf(hv[m].w, ki, hk[3]);
        hq[0] = fmaf(hv[m].x, qi, hq[0]);
        hq[1] = fmaf(hv[m].y, qi, hq[1]);
        hq[2] = fmaf(hv[m].z, qi, hq[2]);
        hq[3] = fmaf(hv[m].w, qi, hq[3]);
        kq = fmaf(ki, qi, kq);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        red_k[rs][4 * cg + c] = hk[c];
        red_q[rs][4 * cg + c] = hq[c];
    }
    if (cg == 0) red_kq[rs] = kq;
    __syncthreads();

    float dl[4];
    float kq_all = 0.f;
#pragma unroll
    for (int p = 0; p < RS; ++p) kq_all += red_kq[p];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = 4 * cg + c;
        float s = 0.f;
#pragma unroll
        for (int p = 0; p < RS; ++p) s += red_k[p][j];
        dl[c] = beta * (Elem<T>::load(a.v, bh * V + j) - alpha * s);
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const float ki = sk[rs + RS * m];
        float4 nv;
        nv.x = fmaf(alpha, hv[m].x, ki * dl[0]);
        nv.y = fmaf(alpha, hv[m].y, ki * dl[1]);
        nv.z = fmaf(alpha, hv[m].z, ki * dl[2]);
        nv.w = fmaf(alpha, hv[m].w, ki * dl[3]);
        store_nt(nv, &st[(rs + RS * m) * CG + cg]);
    }
    if (rs == 0) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = 4 * cg + c;
            float s = 0.f;
#pragma unroll
            for (int p = 0; p < RS; ++p) s += red_q[p][j];
            Elem<T>::store(a.o, bh * V + j, fmaf(alpha, s, dl[c] * kq_all));
        }
    }
}

template <typename T, int K, int V>
hipError_t launch_t(const DecodeArgs &a, hipStream_t s) {
    const int64_t n = (int64_t)a.B * a.H;
    if (n == 0) return hipSuccess;
    constexpr int nt = threads_for<K, V>();
    hipLaunchKernelGGL((decode_step_kernel<T, K, V>), dim3((unsigned)n), dim3(nt), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int K, int V, int dtype, const DecodeArgs &a, hipStream_t s) {
    if (K == 32 && V == 32)
        return dtype == GDN_F32 ? launch_t<float, 32, 32>(a, s) : launch_t<bf16_t, 32, 32>(a, s);
    if (K == 128 && V == 128)
        return dtype == GDN_F32 ? launch_t<float, 128, 128>(a, s) : launch_t<bf16_t, 128, 128>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
