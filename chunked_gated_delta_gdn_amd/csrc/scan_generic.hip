// Chunked gated delta rule on the fp32 vector ALU (any supported shape, fp32
// or bf16 inputs; fp32 arithmetic throughout).
//
// Chunk algebra (MaxText PR "Add context parallelism to the Gated Delta Net",
// section "Why", affine equations for h_out and o, with the symbols read as
// follows; G_r is the within-chunk cumulative log-decay):
//   A[r,s]    = beta_r exp(G_r - G_s) k_r.k_s          (s < r)
//   (I + A) w = diag(beta exp(G)) K,   (I + A) u = diag(beta) V
//   k_tilde_s = exp(G_C - G_s) k_s,    q_g[r] = exp(G_r) q_r
//   attn[r,s] = exp(G_r - G_s) q_r.k_s                  (s <= r)
//   delta     = u - w h
//   o         = q_g h + attn delta
//   h         <- exp(G_C) h + k_tilde^T delta
// The columns of the state are independent under this map, so a workgroup
// owns a group of NCOL columns of X, where X = h (EMIT) or X = [M | h]
// (CARRY: the zero-state pass that also carries M, started from [I | 0], with
// u = 0 on the M columns -- the low-rank update M <- gamma M - k_tilde^T (w M)
// of section "Implementation").  One thread owns one column of X in registers.
//
// This kernel favours plainness over speed: the shared chunk operands sit in
// LDS as fp32, every product is a loop of FMAs.  The bf16 K=V=128 hot path
// runs on the matrix cores instead (scan_mfma.hip).
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

template <typename T, int K, int C>
__device__ __forceinline__ void load_rows(float *dst, int ld, const void *src, int64_t tc,
                                          int L, int H, int h, int width, int col0,
                                          int row_len) {
    // dst[r*ld + i] = src[((tc + r) * H + h) * row_len + col0 + i] for r < L, else 0.
    for (int e = threadIdx.x; e < C * width; e += kThreads) {
        const int r = e / width, i = e % width;
        float val = 0.f;
        if (r < L) val = Elem<T>::load(src, ((tc + r) * H + h) * (int64_t)row_len + col0 + i);
        dst[r * ld + i] = val;
    }
}

template <int C>
__device__ __forceinline__ void load_decay(float *sG, float *sb, const float *g,
                                           const float *beta, int64_t tc, int L, int H, int h) {
    const int r = threadIdx.x;
    if (r < C) {
        const bool ok = r < L;
        sG[r] = ok ? g[(tc + r) * H + h] : 0.f;
        sb[r] = ok ? beta[(tc + r) * H + h] : 0.f;
    }
}

template <int C>
__device__ __forceinline__ void cumsum_decay(float *sG) {
    if (threadIdx.x == 0) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
            acc += sG[r];
            sG[r] = acc;
        }
    }
}

// sa[r*(C+1) + s] = beta_r exp(G_r - G_s) k_r.k_s for s < r, else 0.
template <int K, int C>
__device__ __forceinline__ void build_A(float *sa, const float *sk, const float *sG,
                                        const float *sb) {
    constexpr int KP = K + 1, CP = C + 1;
    for (int p = threadIdx.x; p < C * C; p += kThreads) {
        const int r = p / C, s = p % C;
        float val = 0.f;
        if (s < r) {
            float dot = 0.f;
#pragma unroll 8
            for (int i = 0; i < K; ++i) dot = fmaf(sk[r * KP + i], sk[s * KP + i], dot);
            val = sb[r] * expf(sG[r] - sG[s]) * dot;
        }
        sa[r * CP + s] = val;
    }
}

// Forward substitution (I + A) x = rhs, one column per thread, in place.
// Columns c < K solve for w (rhs beta_r exp(G_r) k[r][c], written to sw);
// columns K .. K+nu-1 solve for u in place on su (rhs beta_r v[r][c]).
template <int K, int C>
__device__ __forceinline__ void solve_wu(float *sw, float *su, int ldu, int nu, const float *sk,
                                         const float *sa, const float *sG, const float *sb) {
    constexpr int KP = K + 1, CP = C + 1;
    for (int c = threadIdx.x; c < K + nu; c += kThreads) {
        if (c < K) {
#pragma unroll 1
            for (int r = 0; r < C; ++r) {
                float acc = sb[r] * expf(sG[r]) * sk[r * KP + c];
                for (int s = 0; s < r; ++s) acc = fmaf(-sa[r * CP + s], sw[s * KP + c], acc);
                sw[r * KP + c] = acc;
            }
        } else {
            const int cc = c - K;
#pragma unroll 1
            for (int r = 0; r < C; ++r) {
                float acc = sb[r] * su[r * ldu + cc];
                for (int s = 0; s < r; ++s) acc = fmaf(-sa[r * CP + s], su[s * ldu + cc], acc);
                su[r * ldu + cc] = acc;
            }
        }
    }
}

template <typename T, int K, int V, int C, int NCOL, bool CARRY, bool WY_IN>
__global__ __launch_bounds__(kThreads) void scan_generic(ScanArgs a) {
    constexpr bool EMIT = !CARRY;
    constexpr int NX = CARRY ? K + V : V;
    constexpr int NG = NX / NCOL;
    constexpr int KP = K + 1, CP = C + 1;
    static_assert(K % NCOL == 0 && V % NCOL == 0 && NCOL <= kThreads, "column groups");
    static_assert(C <= kThreads, "chunk rows");

    __shared__ float sk[C * KP];   // k, then k_tilde
    __shared__ float sw[C * KP];   // w
    __shared__ float sq[EMIT ? C * KP : 1];   // q, then q_g
    __shared__ float su[C * NCOL]; // v, then u (own h columns)
    __shared__ float sa[C * CP];   // A, then attn
    __shared__ float sd[C * NCOL]; // delta (own columns)
    __shared__ float sG[C], sb[C];

    const int tid = threadIdx.x;
    int bid = blockIdx.x;
    const int cg = bid % NG;
    bid /= NG;
    const int H = a.H;
    const int h = bid % H;
    const int chain = bid / H;
    const UnitRef ur = a.ct.packed ? packed_unit(a.ct, chain, h, H, C) : batch_unit(a.ct, chain, h, H, C, CARRY);
    if (ur.carry != CARRY) return;   // an item of the other kind (the host never lists one)
    const ChainSpan sp = ur.sp;
    const int col0 = cg * NCOL;
    const bool is_M = CARRY && col0 < K;
    const int hc0 = CARRY ? col0 - K : col0;
    const int64_t slot = ur.slot;   // state row of h_in (emit) or M_out / U_out (carry)
    const int hk = h / (H / a.Hk);  // key head of this value head (grouped order)
    const bool active = tid < NCOL;

    float x[K];
    if (active) {
        if (CARRY) {
#pragma unroll
            for (int i = 0; i < K; ++i) x[i] = (is_M && i == col0 + tid) ? 1.f : 0.f;
        } else {
            const float *hin = a.h_in;
#pragma unroll
            for (int i = 0; i < K; ++i)
                x[i] = hin ? hin[(slot * K + i) * V + hc0 + tid] : 0.f;
        }
    }

    const int64_t n_chunks = (sp.t1 - sp.t0 + C - 1) / C;
    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t tc = sp.t0 + j * C;
        const int L = (int)((sp.t1 - tc) < C ? (sp.t1 - tc) : C);
        const int64_t chunk = sp.chunk0 + j;

        load_rows<T, K, C>(sk, KP, a.k, tc, L, a.Hk, hk, K, 0, K);
        if (EMIT) load_rows<T, K, C>(sq, KP, a.q, tc, L, a.Hk, hk, K, 0, K);
        if (WY_IN) {
            for (int e = tid; e < C * K; e += kThreads) {
                const int r = e / K, i = e % K;
                sw[r * KP + i] = Elem<T>::load(a.wy_w, ((chunk * H + h) * C + r) * K + i);
            }
            if (!is_M) {
                for (int e = tid; e < C * NCOL; e += kThreads) {
                    const int r = e / NCOL, c = e % NCOL;
                    su[r * NCOL + c] =
                        Elem<T>::load(a.wy_u, ((chunk * H + h) * C + r) * V + hc0 + c);
                }
            }
        } else if (!is_M) {
            load_rows<T, K, C>(su, NCOL, a.v, tc, L, H, h, NCOL, hc0, V);
        }
        load_decay<C>(sG, sb, a.g, a.beta, tc, L, H, h);
        __syncthreads();
        cumsum_decay<C>(sG);
        __syncthreads();

        if (!WY_IN) {
            build_A<K, C>(sa, sk, sG, sb);
            __syncthreads();
            solve_wu<K, C>(sw, su, NCOL, is_M ? 0 : NCOL, sk, sa, sG, sb);
            __syncthreads();
        }
        if (EMIT) {
            for (int p = tid; p < C * C; p += kThreads) {
                const int r = p / C, s = p % C;
                float val = 0.f;
                if (s <= r) {
                    float dot = 0.f;
#pragma unroll 8
                    for (int i = 0; i < K; ++i) dot = fmaf(sq[r * KP + i], sk[s * KP + i], dot);
                    val = expf(sG[r] - sG[s]) * dot;
                }
                sa[r * CP + s] = val;
            }
            __syncthreads();
        }
        const float gC = sG[C - 1];
        for (int e = tid; e < C * K; e += kThreads) {
            const int r = e / K, i = e % K;
            sk[r * KP + i] *= expf(gC - sG[r]);
            if (EMIT) sq[r * KP + i] *= expf(sG[r]);
        }
        __syncthreads();

        if (active) {
#pragma unroll 1
            for (int r = 0; r < C; ++r) {
                float acc = is_M ? 0.f : su[r * NCOL + tid];
#pragma unroll
                for (int i = 0; i < K; ++i) acc = fmaf(-sw[r * KP + i], x[i], acc);
                sd[r * NCOL + tid] = acc;
            }
            if (EMIT) {
#pragma unroll 1
                for (int r = 0; r < L; ++r) {
                    float acc = 0.f;
#pragma unroll
                    for (int i = 0; i < K; ++i) acc = fmaf(sq[r * KP + i], x[i], acc);
                    for (int s = 0; s <= r; ++s) acc = fmaf(sa[r * CP + s], sd[s * NCOL + tid], acc);
                    Elem<T>::store(a.o, ((tc + r) * H + h) * (int64_t)V + hc0 + tid, acc);
                }
            }
            const float gam = expf(gC);
#pragma unroll
            for (int i = 0; i < K; ++i) x[i] *= gam;
#pragma unroll 1
            for (int r = 0; r < C; ++r) {
                const float dl = sd[r * NCOL + tid];
#pragma unroll
                for (int i = 0; i < K; ++i) x[i] = fmaf(sk[r * KP + i], dl, x[i]);
            }
        }
        __syncthreads();
    }

    if (active) {
        if (CARRY) {
            if (is_M) {
#pragma unroll
                for (int i = 0; i < K; ++i) a.M_out[(slot * K + i) * K + col0 + tid] = x[i];
            } else {
#pragma unroll
                for (int i = 0; i < K; ++i) a.U_out[(slot * K + i) * V + hc0 + tid] = x[i];
            }
        } else if (a.h_out && ur.final_state) {
            const int64_t so = ur.out_slot;
#pragma unroll
            for (int i = 0; i < K; ++i) a.h_out[(so * K + i) * V + hc0 + tid] = x[i];
        }
    }
}

// One workgroup per (chunk, head): writes that chunk's w [C,K] and u [C,V].
template <typename T, int K, int V, int C>
__global__ __launch_bounds__(kThreads) void prepare_generic(PrepArgs a) {
    constexpr int KP = K + 1, CP = C + 1;
    __shared__ float sk[C * KP];
    __shared__ float sw[C * KP];
    __shared__ float su[C * V];
    __shared__ float sa[C * CP];
    __shared__ float sG[C], sb[C];

    const int H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    // Locate the chunk's sequence and its first token.
    int64_t tc, tend;
    if (a.ct.packed) {
        int n = 0;
        while (n + 1 < a.ct.n_seqs && a.ct.chunk_start[n + 1] <= chunk) ++n;
        tc = a.ct.seq_start[n] + (chunk - a.ct.chunk_start[n]) * C;
        tend = a.ct.seq_start[n + 1];
    } else {
        const int64_t per = (a.ct.seq_len + C - 1) / C;
        const int64_t n = chunk / per;
        tc = n * a.ct.seq_len + (chunk % per) * C;
        tend = (n + 1) * a.ct.seq_len;
    }
    const int L = (int)((tend - tc) < C ? (tend - tc) : C);

    load_rows<T, K, C>(sk, KP, a.k, tc, L, a.Hk, h / (H / a.Hk), K, 0, K);
    load_rows<T, K, C>(su, V, a.v, tc, L, H, h, V, 0, V);
    load_decay<C>(sG, sb, a.g, a.beta, tc, L, H, h);
    __syncthreads();
    cumsum_decay<C>(sG);
    __syncthreads();
    build_A<K, C>(sa, sk, sG, sb);
    __syncthreads();
    solve_wu<K, C>(sw, su, V, V, sk, sa, sG, sb);
    __syncthreads();
    for (int e = threadIdx.x; e < C * K; e += kThreads) {
        const int r = e / K, i = e % K;
        Elem<T>::store(a.wy_w, ((chunk * H + h) * C + r) * K + i, sw[r * KP + i]);
    }
    for (int e = threadIdx.x; e < C * V; e += kThreads) {
        const int r = e / V, i = e % V;
        Elem<T>::store(a.wy_u, ((chunk * H + h) * C + r) * V + i, su[r * V + i]);
    }
}

template <typename T, int K, int V, int C, int NCOL>
hipError_t launch_scan_t(bool carry, const ScanArgs &a, hipStream_t s) {
    const bool wy = a.wy_w != nullptr;
    const int ng = carry ? (K + V) / NCOL : V / NCOL;
    const dim3 grid((unsigned)((int64_t)a.n_chains * a.H * ng)), block(kThreads);
    if (grid.x == 0) return hipSuccess;
    if (carry) {
        if (wy) hipLaunchKernelGGL((scan_generic<T, K, V, C, NCOL, true, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((scan_generic<T, K, V, C, NCOL, true, false>), grid, block, 0, s, a);
    } else {
        if (wy) hipLaunchKernelGGL((scan_generic<T, K, V, C, NCOL, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((scan_generic<T, K, V, C, NCOL, false, false>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <typename T, int K, int V, int C>
hipError_t launch_prepare_t(const PrepArgs &a, hipStream_t s) {
    const int64_t n = a.n_chunks * a.H;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL((prepare_generic<T, K, V, C>), dim3((unsigned)n), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_generic(int K, int V, int C, int dtype, bool carry, const ScanArgs &a,
                               hipStream_t s) {
    if (K == 32 && V == 32 && C == 16) {
        return dtype == GDN_F32 ? launch_scan_t<float, 32, 32, 16, 32>(carry, a, s)
                                : launch_scan_t<bf16_t, 32, 32, 16, 32>(carry, a, s);
    }
    if (K == 128 && V == 128 && C == 64) {
        return dtype == GDN_F32 ? launch_scan_t<float, 128, 128, 64, 64>(carry, a, s)
                                : launch_scan_t<bf16_t, 128, 128, 64, 64>(carry, a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prepare(int K, int V, int C, int dtype, const PrepArgs &a, hipStream_t s) {
    if (mfma_prepare_available(K, V, C, dtype)) return launch_prepare_mfma(a, s);
    if (K == 32 && V == 32 && C == 16) {
        return dtype == GDN_F32 ? launch_prepare_t<float, 32, 32, 16>(a, s)
                                : launch_prepare_t<bf16_t, 32, 32, 16>(a, s);
    }
    if (K == 128 && V == 128 && C == 64) {
        return dtype == GDN_F32 ? launch_prepare_t<float, 128, 128, 64>(a, s)
                                : launch_prepare_t<bf16_t, 128, 128, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
