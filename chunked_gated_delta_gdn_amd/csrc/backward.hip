// Backward pass of the chunked gated delta rule: the gradients of a loss
// l(o, h_T) with respect to q, k, v, g, beta and h0, given dl/do and dl/dh_T.
//
// The MaxText PR "Add context parallelism to the Gated Delta Net" runs and
// tests a backward pass (section "Tests") but prints no algorithm for it, so
// this is the chain rule taken through the chunk equations of its section
// "Why" (with the symbols read as in the forward kernels):
//   A[r,s] = beta_r D[r,s] k_r.k_s (s < r),  D[r,s] = exp(G_r - G_s),
//   T = (I + A)^{-1},  w = T Kb,  u = T Vb,  Kb = diag(beta exp(G)) K,
//   Vb = diag(beta) V,  delta = u - w h,  o = q_g h + attn delta,
//   h' = gamma h + k_tilde^T delta.
// With h the state at a chunk's start and dh = dl/dh' at its end:
//   ddelta = attn^T do + k_tilde dh
//   dh_in  = gamma dh + q_g^T do - w^T ddelta          (the reverse scan)
//   dattn  = causal(do delta^T),  dw = -ddelta h^T,  du = ddelta
//   dT     = du Vb^T + dw Kb^T,   dVb = T^T du,  dKb = T^T dw
//   dA     = -strict_lower(T^T dT T^T)
// and every chunk quantity passes its gradient on to q, k, v, beta and the
// within-chunk cumulative decay G (dg is the reverse cumulative sum of dG).
//
// Four launches (a fifth sums dq, dk over grouped key heads), all fp32
// arithmetic; at K = V = 128, C = 64 the products run as fp32 matrix-core
// tiles, elsewhere (and for the small shape) on the vector ALU:
//   1. prep   (chunk, head):    T, attn, Dec (.) K K^T, w, u
//   2. states (chain, head, column group), chunks in order: the state at
//      every chunk start and delta
//   3. dstates (chain, head, column group), chunks in reverse: dl/dh at every
//      chunk end and ddelta; dh0 at the end
//   (the stored states are K x V at K = V = 128, transposed V x K elsewhere)
//   4. grads  (chunk, head):    dq, dk, dv, dg, dbeta of the chunk's tokens
// The state columns are independent under both scans (the forward's and its
// reverse), so a workgroup of 2. and 3. owns NCOL of them.
#include "dev_common.h"
#include "gdn_internal.h"
#include "mfma_tile.h"

namespace gdn {
namespace {

struct ChunkLoc {
    int64_t tc;   // first token of the chunk
    int L;        // real tokens in it (rows L .. C-1 are padding)
};

__device__ __forceinline__ ChunkLoc locate_chunk(const ChainTable &ct, int64_t chunk, int C) {
    int64_t tc, tend;
    if (ct.packed) {
        int lo = 0, hi = ct.n_seqs - 1;   // last n with chunk_start[n] <= chunk
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (ct.chunk_start[mid] <= chunk) lo = mid;
            else hi = mid - 1;
        }
        tc = ct.seq_start[lo] + (chunk - ct.chunk_start[lo]) * C;
        tend = ct.seq_start[lo + 1];
    } else {
        const int64_t per = (ct.seq_len + C - 1) / C;
        const int64_t n = chunk / per;
        tc = n * ct.seq_len + (chunk % per) * C;
        tend = (n + 1) * ct.seq_len;
    }
    ChunkLoc l;
    l.tc = tc;
    l.L = (int)((tend - tc) < C ? (tend - tc) : C);
    return l;
}

// Within-chunk cumulative log-decay G of rows 0 .. C-1 (padding rows add 0)
// and the row factors sEg[r] = exp(G_r), sEk[r] = exp(G_{C-1} - G_r), from
// lane r's own g (0 past the chunk).  Called by the 64 lanes of wave 0.
template <int C>
__device__ __forceinline__ void chunk_decay(float x, float *sG, float *sEg, float *sEk) {
    static_assert(C <= 64, "one wave scans the chunk");
    const int lane = threadIdx.x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    const float Gl = __shfl(x, C - 1);
    if (lane < C) {
        sG[lane] = x;
        sEg[lane] = expf(x);
        sEk[lane] = expf(Gl - x);
    }
}

template <int C>
__device__ __forceinline__ void load_cumdecay(float *sG, float *sEg, float *sEk, const float *g,
                                              int64_t tc, int L, int H, int h) {
    if (threadIdx.x < 64)
        chunk_decay<C>(threadIdx.x < C && threadIdx.x < L ? g[(tc + threadIdx.x) * H + h] : 0.f,
                       sG, sEg, sEk);
    __syncthreads();
}

// Adds x, summed over the N consecutive lanes that share `row`, to slot[row],
// where slot is the calling wave's own array: the first of those lanes writes
// it, so a (wave, row) pair must have one writing lane per phase.  Partial
// sums are combined later in a fixed order, so the result does not depend on
// timing (N a power of two; every lane of the wave must call it).
template <int N>
__device__ __forceinline__ void put_row(float *slot, int row, float x) {
    constexpr int W = N < 64 ? N : 64;
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & (W - 1)) == 0) slot[row] += x;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 lds4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// ---------------------------------------------------------------- 1. prep
template <typename T, int K, int V, int C, int NT>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BwdArgs a) {
    constexpr int KP = K + 1, CP = C + 1;
    __shared__ float sk[C * KP], sq[C * KP];
    __shared__ float sA[C * CP], sT[C * CP];
    __shared__ float sv[C * V];   // Vb = diag(beta) V
    __shared__ float sG[C], sEg[C], sEk[C], sb[C], sbg[C];
    const int tid = threadIdx.x, H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    const ChunkLoc cl = locate_chunk(a.ct, chunk, C);
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);   // key head of this value head (grouped order)
    const int64_t ch = chunk * H + h;

    for (int e = tid; e < C * K; e += NT) {
        const int r = e / K, i = e % K;
        const bool ok = r < cl.L;
        const int64_t x = (cl.tc + r) * rowK + hk * K + i;
        sk[r * KP + i] = ok ? Elem<T>::load(a.k, x) : 0.f;
        sq[r * KP + i] = ok ? Elem<T>::load(a.q, x) : 0.f;
    }
    if (tid < C) sb[tid] = tid < cl.L ? a.beta[(cl.tc + tid) * H + h] : 0.f;
    load_cumdecay<C>(sG, sEg, sEk, a.g, cl.tc, cl.L, H, h);
    if (tid < C) sbg[tid] = sb[tid] * sEg[tid];
    for (int e = tid; e < C * V; e += NT) {
        const int r = e / V, j = e % V;
        sv[e] = r < cl.L ? sb[r] * Elem<T>::load(a.v, (cl.tc + r) * rowV + h * V + j) : 0.f;
    }

    float *Ak = a.Ak + ch * C * C, *attn = a.attn + ch * C * C;
    if constexpr (K == 128 && V == 128 && C == 64 && NT == 512) {
        // the Grams K K^T and Q K^T as fp32 matrix-core tiles, two of the 4 x 4
        // per wave (lane (li, lg) gives A[li][k], B[k][li], k = 4 (4 q + lg) + e;
        // it holds D[4 lg + e][li])
        const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
            const int tile = 2 * wv + u2, tr = tile >> 2, tcol = tile & 3;
            const int r = 16 * tr + li, sc = 16 * tcol + li;
            f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qk = kk;
            for (int q = 0; q < 8; ++q) {
                const int i0 = 4 * (4 * q + lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float bk = sk[sc * KP + i0 + e];
                    kk = __builtin_amdgcn_mfma_f32_16x16x4f32(sk[r * KP + i0 + e], bk, kk, 0, 0, 0);
                    qk = __builtin_amdgcn_mfma_f32_16x16x4f32(sq[r * KP + i0 + e], bk, qk, 0, 0, 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * tr + 4 * lg + e;
                const float dec = sc <= rr ? expf(sG[rr] - sG[sc]) : 0.f;
                const float ak = sc < rr ? dec * kk[e] : 0.f;
                sA[rr * CP + sc] = sb[rr] * ak;   // A itself
                Ak[rr * C + sc] = ak;
                attn[rr * C + sc] = dec * qk[e];
            }
        }
    } else {
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s = e % C;
            float kk = 0.f, qk = 0.f, dec = 0.f;
            if (s <= r) {
                for (int i = 0; i < K; ++i) {
                    kk = fmaf(sk[r * KP + i], sk[s * KP + i], kk);
                    qk = fmaf(sq[r * KP + i], sk[s * KP + i], qk);
                }
                dec = expf(sG[r] - sG[s]);
            }
            const float ak = s < r ? dec * kk : 0.f;
            sA[r * CP + s] = sb[r] * ak;   // A itself
            Ak[e] = ak;
            attn[e] = dec * qk;
        }
    }
    __syncthreads();
    // T = (I + A)^{-1} by forward substitution, row by row: column c belongs to
    // the PARTS consecutive lanes c * PARTS .., each summing every PARTS-th term
    {
        constexpr int PARTS = NT / C;
        static_assert(PARTS * C == NT && (PARTS & (PARTS - 1)) == 0 && PARTS <= 64, "solve lanes");
        const int c = tid / PARTS, part = tid % PARTS;
        for (int r = 0; r < C; ++r) {
            float x = 0.f;
            if (r > c)
                for (int s = c + part; s < r; s += PARTS) x = fmaf(-sA[r * CP + s], sT[s * CP + c], x);
#pragma unroll
            for (int off = PARTS / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
            if (part == 0) sT[r * CP + c] = r == c ? 1.f : (r > c ? x : 0.f);
            __syncthreads();
        }
    }
    float *To = a.T + ch * C * C, *w = a.w + ch * C * K, *u = a.u + ch * C * V;
    for (int e = tid; e < C * C; e += NT) To[e] = sT[(e / C) * CP + e % C];
    if constexpr (K == 128 && V == 128 && C == 64 && NT == 512) {
        // w = T diag(beta exp(G)) K and u = T diag(beta) V: wave wv owns column
        // tile wv of both and the four row tiles
        const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
        const int col = 16 * wv + li;
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 aw[4] = {z4, z4, z4, z4}, au[4] = {z4, z4, z4, z4};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s0 = 4 * (4 * q + lg);
            float bw[4], bu[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bw[e] = sbg[s0 + e] * sk[(s0 + e) * KP + col];
                bu[e] = sv[(s0 + e) * V + col];
            }
#pragma unroll
            for (int tr = 0; tr < 4; ++tr)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ta = sT[(16 * tr + li) * CP + s0 + e];
                    aw[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta, bw[e], aw[tr], 0, 0, 0);
                    au[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta, bu[e], au[tr], 0, 0, 0);
                }
        }
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                w[r * K + col] = aw[tr][e];
                u[r * V + col] = au[tr][e];
            }
    } else {
        for (int e = tid; e < C * K; e += NT) {
            const int r = e / K, i = e % K;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc = fmaf(sT[r * CP + s], sbg[s] * sk[s * KP + i], acc);
            w[e] = acc;
        }
        for (int e = tid; e < C * V; e += NT) {
            const int r = e / V, j = e % V;
            float acc = 0.f;
            for (int s = 0; s <= r; ++s) acc = fmaf(sT[r * CP + s], sv[s * V + j], acc);
            u[e] = acc;
        }
    }
}

// ------------------------------------------------ 1b. prep, K = V = 128, C = 64, bf16
// The same per-chunk quantities as bwd_prep_kernel, for bf16 inputs.  k, q and
// v are kept in LDS as the bf16 values they are, so the Grams K K^T and Q K^T
// run on the bf16 matrix cores with fp32 accumulation: every product of two
// bf16 values is exact in fp32, so only the order of the fp32 sums differs
// from an fp32 evaluation.  T = (I + A)^{-1} is formed blockwise over 16 x 16
// blocks: the four diagonal blocks by forward substitution (one lane per
// column), then T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj one block diagonal at
// a time, on the fp32 matrix cores -- three dependent levels instead of 64
// dependent rows.  The LDS footprint (about 70 KB) lets two chunks share a CU.
template <typename T>
__global__ __launch_bounds__(512) void bwd_prep_mfma_kernel(BwdArgs a) {
    static_assert(sizeof(typename Elem<T>::raw_t) == 2, "k, q, v are kept as bf16");
    constexpr int K = 128, V = 128, C = 64, NT = 512;
    constexpr int RS = K + 8;   // bf16 rows [C][RS], 16-byte aligned
    constexpr int CP = C + 1;   // fp32 rows of C x C tiles
    typedef uint16_t u16;
    __shared__ __attribute__((aligned(16))) u16 sk[C * RS];
    __shared__ __attribute__((aligned(16))) u16 sv[C * RS];
    __shared__ __attribute__((aligned(16))) float RQ[C * RS / 2];   // q rows (bf16), then T [C][CP]
    __shared__ float sA[C * CP];
    __shared__ float sG[C], sEg[C], sEk[C], sb[C], sbg[C];
    static_assert(C * CP <= C * RS / 2 && (RS * 2) % 16 == 0, "T fits where q was");
    u16 *const sq = reinterpret_cast<u16 *>(RQ);
    float *const sT = RQ;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    const ChunkLoc cl = locate_chunk(a.ct, chunk, C);
    const int L = cl.L;
    const int64_t tc = cl.tc;
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);
    const int64_t ch = chunk * H + h;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    auto bf = [](u16 x) { return __uint_as_float((uint32_t)x << 16); };

    // rows of k, q, v (rows past L zero), 16 bytes per load
#pragma unroll
    for (int m = 0; m < (C * K / 8) / NT; ++m) {
        const int e8 = tid + NT * m, r = (8 * e8) / K, j = (8 * e8) % K;
        const int64_t rr = tc + min(r, L - 1);
        uint4 wk = *reinterpret_cast<const uint4 *>(static_cast<const u16 *>(a.k) + rr * rowK + hk * K + j);
        uint4 wq = *reinterpret_cast<const uint4 *>(static_cast<const u16 *>(a.q) + rr * rowK + hk * K + j);
        uint4 wvv = *reinterpret_cast<const uint4 *>(static_cast<const u16 *>(a.v) + rr * rowV + h * V + j);
        if (r >= L) wk = wq = wvv = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(&sk[r * RS + j]) = wk;
        *reinterpret_cast<uint4 *>(&sq[r * RS + j]) = wq;
        *reinterpret_cast<uint4 *>(&sv[r * RS + j]) = wvv;
    }
    if (tid < C) sb[tid] = tid < L ? a.beta[(tc + tid) * H + h] : 0.f;
    load_cumdecay<C>(sG, sEg, sEk, a.g, tc, L, H, h);   // (synchronises)
    if (tid < C) sbg[tid] = sb[tid] * sEg[tid];

    // ---- Grams: wave wv owns tiles 2 wv, 2 wv + 1 of the 4 x 4; a 16 x 16 x 32
    // bf16 product takes 8 consecutive k of a row from each lane
    float *Ak = a.Ak + ch * C * C, *attn = a.attn + ch * C * C;
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
        const int tile = 2 * wv + u2, tr = tile >> 2, tcol = tile & 3;
        f32x4 kk = z4, qk = z4;
        if (tcol <= tr) {
            const int r = 16 * tr + li, sc = 16 * tcol + li;
#pragma unroll
            for (int kb = 0; kb < K / 32; ++kb) {
                const int o = 32 * kb + 8 * lg;
                const mfma::bf16x8 b = mfma::as8(*reinterpret_cast<const uint4 *>(&sk[sc * RS + o]));
                kk = mfma::mma32(mfma::as8(*reinterpret_cast<const uint4 *>(&sk[r * RS + o])), b, kk);
                qk = mfma::mma32(mfma::as8(*reinterpret_cast<const uint4 *>(&sq[r * RS + o])), b, qk);
            }
        }
        const int sc = 16 * tcol + li;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 16 * tr + 4 * lg + e;
            const float dec = sc <= rr ? expf(sG[rr] - sG[sc]) : 0.f;
            const float ak = sc < rr ? dec * kk[e] : 0.f;
            sA[rr * CP + sc] = sb[rr] * ak;   // A itself
            Ak[rr * C + sc] = ak;
            attn[rr * C + sc] = dec * qk[e];
        }
    }
    __syncthreads();   // sq is dead from here: sT takes its place

    // ---- diagonal blocks: lane 16 b + c of wave 0 forms column c of T_bb;
    // the other waves clear the blocks above the diagonal
    if (wv == 0) {
        const int b = lane >> 4, c = lane & 15;
        const float *Ab = sA + 16 * b * CP + 16 * b;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = r == c ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < r; ++s2) x = fmaf(-Ab[r * CP + s2], t[s2], x);
            t[r] = x;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sT[(16 * b + r) * CP + 16 * b + c] = t[r];
    } else {
        for (int e = tid - 64; e < 6 * 256; e += NT - 64) {
            const int blk = e >> 8, w = e & 255;   // blocks (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
            const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
            const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
            sT[(16 * bi + (w >> 4)) * CP + 16 * bj + (w & 15)] = 0.f;
        }
    }
    __syncthreads();
    // ---- below the diagonal, one block diagonal per level:
    // T_ij = -T_ii (sum_{m=j}^{i-1} A_im T_mj)
    auto off_block = [&](int i, int j) {
        f32x4 P = z4;
        for (int m = j; m < i; ++m)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                P = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * i + li) * CP + 16 * m + 4 * kk + lg],
                                                         sT[(16 * m + 4 * kk + lg) * CP + 16 * j + li], P, 0, 0, 0);
        // P is held as P[4 lg + e][li]: step e of the second product sums
        // over k = 4 lg + e
        f32x4 R = z4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            R = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * i + li) * CP + 16 * i + 4 * lg + e], P[e], R, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * i + 4 * lg + e) * CP + 16 * j + li] = -R[e];
    };
#pragma unroll
    for (int lvl = 1; lvl < 4; ++lvl) {
        if (wv < 4 - lvl) off_block(wv + lvl, wv);
        __syncthreads();
    }

    // ---- T out; w = T diag(beta exp(G)) K and u = T diag(beta) V: wave wv owns
    // column tile wv of both and the four row tiles (T's zero blocks skipped)
    float *To = a.T + ch * C * C, *w = a.w + ch * C * K, *u = a.u + ch * C * V;
#pragma unroll
    for (int m = 0; m < (C * C) / NT; ++m) {
        const int e = tid + NT * m;
        To[e] = sT[(e / C) * CP + e % C];
    }
    {
        const int col = 16 * wv + li;
        f32x4 aw[4] = {z4, z4, z4, z4}, au[4] = {z4, z4, z4, z4};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s0 = 4 * (4 * q + lg);
            float bw[4], bu[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bw[e] = sbg[s0 + e] * bf(sk[(s0 + e) * RS + col]);
                bu[e] = sb[s0 + e] * bf(sv[(s0 + e) * RS + col]);
            }
#pragma unroll
            for (int tr = q; tr < 4; ++tr)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ta = sT[(16 * tr + li) * CP + s0 + e];
                    aw[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta, bw[e], aw[tr], 0, 0, 0);
                    au[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(ta, bu[e], au[tr], 0, 0, 0);
                }
        }
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                w[r * K + col] = aw[tr][e];
                u[r * V + col] = au[tr][e];
            }
    }
}

// ---------------------------------------------------------------- 2. states
// First token tc and real length L of chunk c of the chain [t0, t1).  The
// scans load a chunk's operands into registers one chunk ahead of their use.
template <int C>
__device__ __forceinline__ void chunk_rows(int64_t t0, int64_t t1, int64_t c, int &L, int64_t &tc) {
    tc = t0 + c * C;
    L = (int)((t1 - tc) < C ? (t1 - tc) : C);
}

// The state a chain's forward scan starts from (h0 of its sequence, or the
// composed state of the chain before it), and the gradient its reverse scan
// starts from (dhT, or the composed gradient of the chain after it); NULL =
// zero.  [K, V] row-major.
__device__ __forceinline__ const float *chain_h_start(const BwdArgs &a, const ChainPos &cp, int h, int64_t KV) {
    if (!cp.first) return a.h_in + (cp.slot * a.H + h) * KV;
    return a.h0 ? a.h0 + ((int64_t)cp.seq * a.H + h) * KV : nullptr;
}
__device__ __forceinline__ const float *chain_dh_end(const BwdArgs &a, const ChainPos &cp, int h, int64_t KV) {
    if (!cp.last) return a.dh_in + (cp.slot * a.H + h) * KV;
    return a.dhT ? a.dhT + ((int64_t)cp.seq * a.H + h) * KV : nullptr;
}

template <typename T, int K, int V, int C, int NCOL, int NT>
__global__ __launch_bounds__(NT) void bwd_states_kernel(BwdArgs a) {
    constexpr int KP = K + 1, NP = NCOL + 1, NG = V / NCOL, EPT = K * NCOL / NT, LPT = C * K / NT;
    static_assert(V % NCOL == 0 && (K * NCOL) % NT == 0 && (C * K) % NT == 0, "column groups");
    static_assert(K % NCOL == 0, "strips of M");
    constexpr int NGK = K / NCOL;
    __shared__ float sw[C * KP], sk[C * KP], sh[K * NP], sd[C * NP];
    __shared__ float sG[C], sEg[C], sEk[C];
    const int tid = threadIdx.x, H = a.H;
    // carry launches add NGK strips of M (identity start, u taken as 0)
    const int ng = a.carry ? NGK + NG : NG;
    const int cg = blockIdx.x % ng, h = (blockIdx.x / ng) % H, n = blockIdx.x / (ng * H);
    const ChainPos cp = chain_pos(a.ct, n, a.N);
    const bool is_M = a.carry && cg < NGK;
    // carries: M of every chain of a split sequence (the forward compose uses
    // all but the last, the reverse one all but the first), U of all but the last
    if (a.carry && (cp.first && cp.last || (!is_M && cp.last))) return;
    const int j0 = (is_M ? cg : cg - (a.carry ? NGK : 0)) * NCOL;
    const ChainSpan sp = chain_span(a.ct, n, C);
    const int64_t rowK = (int64_t)a.Hk * K;
    const int hk = h / (H / a.Hk);
    const int64_t KV = (int64_t)K * V;

    float hr[EPT];
    const float *hst = a.carry ? nullptr : chain_h_start(a, cp, h, KV);
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + NT * m, i = e % K, jj = e / K;
        hr[m] = is_M ? (i == j0 + jj ? 1.f : 0.f) : hst ? hst[(int64_t)i * V + j0 + jj] : 0.f;
    }
    const int64_t nch = (sp.t1 - sp.t0 + C - 1) / C;
    // w, raw k and g of the next chunk, fetched while the current one computes
    float pw[LPT], pk[LPT], pg = 0.f;
    auto fetch = [&](int64_t c) {
        int L;
        int64_t tc;
        chunk_rows<C>(sp.t0, sp.t1, c, L, tc);
        const float *w = a.w + ((sp.chunk0 + c) * H + h) * C * K;
#pragma unroll
        for (int m = 0; m < LPT; ++m) {
            const int e = tid + NT * m, r = e / K, i = e % K;
            pw[m] = w[e];
            pk[m] = r < L ? Elem<T>::load(a.k, (tc + r) * rowK + hk * K + i) : 0.f;
        }
        pg = tid < C && tid < L ? a.g[(tc + tid) * H + h] : 0.f;
    };
    if (nch > 0) fetch(0);
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t ch = (sp.chunk0 + c) * H + h;
        float *hs = a.hs + ch * KV;
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            if (!a.carry) hs[(int64_t)(j0 + jj) * K + i] = hr[m];
            sh[i * NP + jj] = hr[m];
        }
#pragma unroll
        for (int m = 0; m < LPT; ++m) {
            const int e = tid + NT * m, r = e / K, i = e % K;
            sw[r * KP + i] = pw[m];
            sk[r * KP + i] = pk[m];
        }
        if (tid < 64) chunk_decay<C>(pg, sG, sEg, sEk);
        __syncthreads();
        if (c + 1 < nch) fetch(c + 1);
        const float gamma = sEg[C - 1];
        const float *u = a.u + ch * C * V;
        float *d = a.d + ch * C * V;
        // delta = u - w h (own columns); k_tilde^T delta = k^T (exp(G_C - G) delta)
        for (int o = tid; o < C * NCOL; o += NT) {
            const int r = o / NCOL, jj = o % NCOL;
            float acc = is_M ? 0.f : u[r * V + j0 + jj];
#pragma unroll 8
            for (int i = 0; i < K; ++i) acc = fmaf(-sw[r * KP + i], sh[i * NP + jj], acc);
            sd[r * NP + jj] = sEk[r] * acc;
            if (!a.carry) d[r * V + j0 + jj] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            float acc = gamma * hr[m];
#pragma unroll 8
            for (int r = 0; r < C; ++r) acc = fmaf(sk[r * KP + i], sd[r * NP + jj], acc);
            hr[m] = acc;
        }
        __syncthreads();
    }
    if (a.carry) {
        const int64_t row = cp.slot * H + h;
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            if (is_M) {
                a.M[row * K * K + (int64_t)i * K + j0 + jj] = hr[m];
                a.Mt[row * K * K + (int64_t)(j0 + jj) * K + i] = hr[m];
            } else {
                a.U[row * KV + (int64_t)i * V + j0 + jj] = hr[m];
            }
        }
    }
}

// ---------------------------------------------------------------- 3. dstates
template <typename T, int K, int V, int C, int NCOL, int NT>
__global__ __launch_bounds__(NT) void bwd_dstates_kernel(BwdArgs a) {
    constexpr int KP = K + 1, CP = C + 1, NP = NCOL + 1, NG = V / NCOL, EPT = K * NCOL / NT;
    constexpr int LPT = C * K / NT, APT = C * C / NT, DPT = (C * NCOL + NT - 1) / NT;
    static_assert(V % NCOL == 0 && (K * NCOL) % NT == 0 && (C * K) % NT == 0 && (C * C) % NT == 0,
                  "column groups");
    __shared__ float sw[C * KP], sk[C * KP], sq[C * KP], sa[C * CP];
    __shared__ float sdh[K * NP], sdo[C * NP], sdoG[C * NP], sdd[C * NP];
    __shared__ float sG[C], sEg[C], sEk[C];
    const int tid = threadIdx.x, H = a.H;
    const int cg = blockIdx.x % NG, h = (blockIdx.x / NG) % H, n = blockIdx.x / (NG * H);
    const int j0 = cg * NCOL;
    const ChainPos cp = chain_pos(a.ct, n, a.N);
    if (a.carry && cp.first) return;   // (carry: zero gradient at the chain's end)
    const ChainSpan sp = chain_span(a.ct, n, C);
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);
    const int64_t KV = (int64_t)K * V;

    float dh[EPT];
    const float *dst = a.carry ? nullptr : chain_dh_end(a, cp, h, KV);
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + NT * m, i = e % K, jj = e / K;
        dh[m] = dst ? dst[(int64_t)i * V + j0 + jj] : 0.f;
    }
    const int64_t nch = (sp.t1 - sp.t0 + C - 1) / C;
    // the next chunk's (in reverse order) w, raw k and q, attn, do columns and g
    float pw[LPT], pk[LPT], pq[LPT], pa[APT], pd[DPT], pg = 0.f;
    auto fetch = [&](int64_t c) {
        int L;
        int64_t tc;
        chunk_rows<C>(sp.t0, sp.t1, c, L, tc);
        const int64_t ch = (sp.chunk0 + c) * H + h;
        const float *w = a.w + ch * C * K, *attn = a.attn + ch * C * C;
#pragma unroll
        for (int m = 0; m < LPT; ++m) {
            const int e = tid + NT * m, r = e / K, i = e % K;
            const bool ok = r < L;
            const int64_t x = (tc + r) * rowK + hk * K + i;
            pw[m] = w[e];
            pk[m] = ok ? Elem<T>::load(a.k, x) : 0.f;
            pq[m] = ok ? Elem<T>::load(a.q, x) : 0.f;
        }
#pragma unroll
        for (int m = 0; m < APT; ++m) pa[m] = attn[tid + NT * m];
#pragma unroll
        for (int m = 0; m < DPT; ++m) {
            const int e = tid + NT * m, r = e / NCOL, jj = e % NCOL;
            pd[m] = e < C * NCOL && r < L ? Elem<T>::load(a.dout, (tc + r) * rowV + h * V + j0 + jj) : 0.f;
        }
        pg = tid < C && tid < L ? a.g[(tc + tid) * H + h] : 0.f;
    };
    if (nch > 0) fetch(nch - 1);
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t ch = (sp.chunk0 + c) * H + h;
        float *dhs = a.dhs + ch * KV;
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            if (!a.carry) dhs[(int64_t)(j0 + jj) * K + i] = dh[m];
            sdh[i * NP + jj] = dh[m];
        }
#pragma unroll
        for (int m = 0; m < LPT; ++m) {
            const int e = tid + NT * m, r = e / K, i = e % K;
            sw[r * KP + i] = pw[m];
            sk[r * KP + i] = pk[m];
            sq[r * KP + i] = pq[m];
        }
#pragma unroll
        for (int m = 0; m < APT; ++m) {
            const int e = tid + NT * m;
            sa[(e / C) * CP + e % C] = pa[m];
        }
#pragma unroll
        for (int m = 0; m < DPT; ++m) {
            const int e = tid + NT * m;
            if (e < C * NCOL) sdo[(e / NCOL) * NP + e % NCOL] = pd[m];
        }
        if (tid < 64) chunk_decay<C>(pg, sG, sEg, sEk);
        __syncthreads();
        if (c > 0) fetch(c - 1);
        const float gamma = sEg[C - 1];
        float *dd = a.dd + ch * C * V;
        // ddelta = attn^T do + k_tilde dh;  also exp(G) do for the q_g^T do term
        for (int o = tid; o < C * NCOL; o += NT) {
            const int r = o / NCOL, jj = o % NCOL;
            float acc = 0.f, acck = 0.f;
#pragma unroll 8
            for (int t = r; t < C; ++t) acc = fmaf(sa[t * CP + r], sdo[t * NP + jj], acc);
#pragma unroll 8
            for (int i = 0; i < K; ++i) acck = fmaf(sk[r * KP + i], sdh[i * NP + jj], acck);
            acc = fmaf(sEk[r], acck, acc);
            sdd[r * NP + jj] = acc;
            sdoG[r * NP + jj] = sEg[r] * sdo[r * NP + jj];
            if (!a.carry) dd[r * V + j0 + jj] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            float acc = gamma * dh[m];
#pragma unroll 8
            for (int r = 0; r < C; ++r) {
                acc = fmaf(sq[r * KP + i], sdoG[r * NP + jj], acc);
                acc = fmaf(-sw[r * KP + i], sdd[r * NP + jj], acc);
            }
            dh[m] = acc;
        }
        __syncthreads();
    }
    float *out = a.carry ? a.E + (cp.slot * H + h) * KV
                         : (a.dh0 && cp.first ? a.dh0 + ((int64_t)cp.seq * H + h) * KV : nullptr);
    if (out) {
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            out[(int64_t)i * V + j0 + jj] = dh[m];
        }
    }
}

// ---------------------------------------------------------------- 2b/3b. the scans on fp32 matrix cores
// K = V = 128, C = 64, a 16-column strip per workgroup of 8 waves.  The
// products are v_mfma_f32_16x16x4_f32 tiles (fp32 in, fp32 accumulate, so the
// arithmetic class is that of the vector kernels above).  For one product
// D += A B, lane (li, lg) = (lane & 15, lane >> 4) gives A[li][k] and B[k][li]
// with k = 4 (4 q + lg) + e at step (q, e), so that its operands for one q are
// 16-byte runs of a row of A and of a row of B^T; it holds D[4 lg + e][li].
// Wave wv owns rows 16 wv .. 16 wv + 15 of the strip (of the state, or of its
// gradient) in that layout.
// Block b of a state-scan launch over units (chain, head) x ng column strips:
// the strips of a unit are 8 block ids apart, so that round-robin dispatch puts
// them on one XCD and their shared reads of the chunk operands meet in that
// XCD's L2.  The grid is padded to whole groups of 8 units (strip_grid);
// padding blocks return false.
__host__ __device__ inline int64_t strip_grid(int64_t units, int ng) { return (units + 7) / 8 * 8 * ng; }
__device__ __forceinline__ bool strip_of_block(int b, int ng, int n_units, int &unit, int &strip) {
    const int grp = b / (8 * ng), rem = b % (8 * ng);
    strip = rem / 8;
    unit = grp * 8 + rem % 8;
    return unit < n_units;
}

template <typename T>
__global__ __launch_bounds__(512) void bwd_states_mfma_kernel(BwdArgs a) {
    constexpr int K = 128, V = 128, C = 64, NCOL = 16, NT = 512, NG = V / NCOL, NGK = K / NCOL;
    constexpr int LDK = K + 4, LDC = C + 4, KPT = C * K / NT;
    __shared__ __attribute__((aligned(16))) float hT[NCOL * LDK];   // state strip [column][row]
    __shared__ __attribute__((aligned(16))) float kT[K * LDC];      // raw k [i][r]
    __shared__ __attribute__((aligned(16))) float dT[NCOL * LDC];   // exp(G_C - G_r) delta [column][r]
    __shared__ float sG[C], sEg[C], sEk[C];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
    const int H = a.H;
    // carry launches add NGK strips of M (identity start, u taken as 0)
    const int ng = a.carry ? NGK + NG : NG;
    int unit, cg;
    if (!strip_of_block((int)blockIdx.x, ng, a.n_units, unit, cg)) return;
    const int h = unit % H, n = unit / H;
    const ChainPos cp = chain_pos(a.ct, n, a.N);
    const bool is_M = a.carry && cg < NGK;
    // carries: M of every chain of a split sequence (the forward compose uses
    // all but the last, the reverse one all but the first), U of all but the last
    if (a.carry && (cp.first && cp.last || (!is_M && cp.last))) return;
    const int j0 = (is_M ? cg : cg - (a.carry ? NGK : 0)) * NCOL;
    const ChainSpan sp = chain_span(a.ct, n, C);
    const int64_t rowK = (int64_t)a.Hk * K;
    const int hk = h / (H / a.Hk);
    const int64_t KV = (int64_t)K * V;
    const int row0 = 16 * wv + 4 * lg;   // this lane's rows of the strip: row0 .. row0 + 3

    f32x4 hacc;
    const float *hst = a.carry ? nullptr : chain_h_start(a, cp, h, KV);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        hacc[e] = is_M ? (row0 + e == j0 + li ? 1.f : 0.f) : hst ? hst[(int64_t)(row0 + e) * V + j0 + li] : 0.f;
    const int64_t nch = (sp.t1 - sp.t0 + C - 1) / C;
    // next chunk: w rows (A operands of delta, waves 0-3), u seeds, raw k, g.
    // Rows past the chunk end are loaded from its last row (every address
    // valid) and zeroed where they are used, a chunk later: a load whose value
    // is masked or converted at once would make the wave wait for it here.
    f32x4 pw[8];
    float pu[4], pg = 0.f;
    // k: 8 consecutive elements of row 16 rb + li at column 32 cb + 8 lg per
    // load, (rb, cb) = (s & 3, s >> 2) for s = 2 wv + m (16 loads of 64 lanes
    // cover the 64 x 128 tile)
    Raw8<T> pk[KPT / 8];
    int pL = 0;
    auto krow = [&](int m) { return 16 * ((2 * wv + m) & 3) + li; };
    auto kcol = [&](int m) { return 32 * ((2 * wv + m) >> 2) + 8 * lg; };
    auto fetch = [&](int64_t c) {
        int L;
        int64_t tc;
        chunk_rows<C>(sp.t0, sp.t1, c, L, tc);
        const int64_t ch = (sp.chunk0 + c) * H + h;
        if (wv < 4) {
            const float *w = a.w + ch * C * K + (16 * wv + li) * K;
#pragma unroll
            for (int q = 0; q < 8; ++q) pw[q] = *reinterpret_cast<const f32x4 *>(w + 4 * (4 * q + lg));
            const float *u = a.u + ch * C * V;
#pragma unroll
            for (int e = 0; e < 4; ++e) pu[e] = is_M ? 0.f : u[(row0 + e) * V + j0 + li];
        }
#pragma unroll
        for (int m = 0; m < KPT / 8; ++m) pk[m].load(a.k, (tc + min(krow(m), L - 1)) * rowK + hk * K + kcol(m));
        pg = a.g[(tc + min(tid, L - 1)) * H + h];
        pL = L;
    };
    if (nch > 0) fetch(0);
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t ch = (sp.chunk0 + c) * H + h;
        if (!a.carry)   // [K][V], the layout the grads kernels read
#pragma unroll
            for (int e = 0; e < 4; ++e) a.hs[ch * KV + (int64_t)(row0 + e) * V + j0 + li] = hacc[e];
        *reinterpret_cast<f32x4 *>(&hT[li * LDK + row0]) = hacc;
#pragma unroll
        for (int m = 0; m < KPT / 8; ++m) {
            const int r = krow(m), i0 = kcol(m);
#pragma unroll
            for (int j = 0; j < 8; ++j) kT[(i0 + j) * LDC + r] = r < pL ? pk[m].at(j) : 0.f;
        }
        if (tid < 64) chunk_decay<C>(tid < C && tid < pL ? pg : 0.f, sG, sEg, sEk);
        __syncthreads();
        f32x4 wc[8];
        float uc[4];
#pragma unroll
        for (int q = 0; q < 8; ++q) wc[q] = pw[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) uc[e] = pu[e];
        if (c + 1 < nch) fetch(c + 1);
        if (wv < 4) {
            // delta rows 16 wv .. of the strip: u - w h
            f32x4 acc = {uc[0], uc[1], uc[2], uc[3]};
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f32x4 hb = lds4(&hT[li * LDK + 4 * (4 * q + lg)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-wc[q][e], hb[e], acc, 0, 0, 0);
            }
            float *d = a.d + ch * C * V;
            f32x4 sc;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (!a.carry) d[(row0 + e) * V + j0 + li] = acc[e];
                sc[e] = sEk[row0 + e] * acc[e];
            }
            *reinterpret_cast<f32x4 *>(&dT[li * LDC + row0]) = sc;
        }
        __syncthreads();
        // h <- gamma h + k^T (exp(G_C - G) delta)
        hacc *= sEg[C - 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 ka = lds4(&kT[(16 * wv + li) * LDC + 4 * (4 * q + lg)]);
            const f32x4 db = lds4(&dT[li * LDC + 4 * (4 * q + lg)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) hacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], db[e], hacc, 0, 0, 0);
        }
        __syncthreads();
    }
    if (a.carry) {
        const int64_t row = cp.slot * H + h;
        if (is_M) {
#pragma unroll
            for (int e = 0; e < 4; ++e) a.M[row * K * K + (int64_t)(row0 + e) * K + j0 + li] = hacc[e];
            *reinterpret_cast<f32x4 *>(a.Mt + row * K * K + (int64_t)(j0 + li) * K + row0) = hacc;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) a.U[row * KV + (int64_t)(row0 + e) * V + j0 + li] = hacc[e];
        }
    }
}

template <typename T>
__global__ __launch_bounds__(512) void bwd_dstates_mfma_kernel(BwdArgs a) {
    constexpr int K = 128, V = 128, C = 64, NCOL = 16, NT = 512, NG = V / NCOL;
    constexpr int LDK = K + 4, LDC = C + 4, KPT = C * K / NT, APT = C * C / NT, DPT = C * NCOL / NT;
    __shared__ __attribute__((aligned(16))) float dhT[NCOL * LDK];   // gradient strip [column][row]
    __shared__ __attribute__((aligned(16))) float sk[C * LDK];       // raw k [r][i]
    __shared__ __attribute__((aligned(16))) float qT[K * LDC];       // raw q [i][r]
    __shared__ __attribute__((aligned(16))) float wT[K * LDC];       // w [i][r]
    __shared__ __attribute__((aligned(16))) float aT[C * LDC];       // attn^T [r][t]
    __shared__ __attribute__((aligned(16))) float doT[NCOL * LDC];   // do strip [column][t]
    __shared__ __attribute__((aligned(16))) float doGT[NCOL * LDC];  // exp(G_t) do [column][t]
    __shared__ __attribute__((aligned(16))) float ddT[NCOL * LDC];   // ddelta [column][r]
    __shared__ float sG[C], sEg[C], sEk[C];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
    const int H = a.H;
    int unit, cg;
    if (!strip_of_block((int)blockIdx.x, NG, a.n_units, unit, cg)) return;
    const int h = unit % H, n = unit / H;
    const int j0 = cg * NCOL;
    const ChainPos cp = chain_pos(a.ct, n, a.N);
    if (a.carry && cp.first) return;   // (carry: zero gradient at the chain's end)
    const ChainSpan sp = chain_span(a.ct, n, C);
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);
    const int64_t KV = (int64_t)K * V;
    const int row0 = 16 * wv + 4 * lg;

    f32x4 dacc;
    const float *dst = a.carry ? nullptr : chain_dh_end(a, cp, h, KV);
#pragma unroll
    for (int e = 0; e < 4; ++e) dacc[e] = dst ? dst[(int64_t)(row0 + e) * V + j0 + li] : 0.f;
    const int64_t nch = (sp.t1 - sp.t0 + C - 1) / C;
    // the previous chunk's operands, fetched a chunk ahead (rows past the chunk
    // end loaded from its last row and zeroed where used, as in the states scan)
    // k, q: 8 consecutive elements of row 16 rb + li at column 32 cb + 8 lg per
    // load, (rb, cb) = (s & 3, s >> 2) for s = 2 wv + m; w (fp32 [C][K]): 4 of row
    // 16 rb + li at column 16 cb + 4 lg, (rb, cb) = (s & 3, s >> 2) for s = 4 wv + m;
    // attn ([C][C]): 4 of row 16 tb + li at column 16 sb + 4 lg for s = 2 wv + m
    Raw8<T> pk[KPT / 8], pq[KPT / 8];
    typename Elem<T>::raw_t pd[DPT];
    f32x4 pw[KPT / 4], pa[APT / 4];
    float pg = 0.f;
    int pL = 0;
    auto krow = [&](int m) { return 16 * ((2 * wv + m) & 3) + li; };
    auto kcol = [&](int m) { return 32 * ((2 * wv + m) >> 2) + 8 * lg; };
    auto wrow = [&](int m) { return 16 * ((4 * wv + m) & 3) + li; };
    auto wcol = [&](int m) { return 16 * ((4 * wv + m) >> 2) + 4 * lg; };
    auto acol = [&](int m) { return 16 * ((2 * wv + m) >> 2) + 4 * lg; };   // (attn rows: krow)
    auto fetch = [&](int64_t c) {
        int L;
        int64_t tc;
        chunk_rows<C>(sp.t0, sp.t1, c, L, tc);
        const int64_t ch = (sp.chunk0 + c) * H + h;
        const float *w = a.w + ch * C * K, *attn = a.attn + ch * C * C;
#pragma unroll
        for (int m = 0; m < KPT / 8; ++m) {
            const int64_t x = (tc + min(krow(m), L - 1)) * rowK + hk * K + kcol(m);
            pk[m].load(a.k, x);
            pq[m].load(a.q, x);
        }
#pragma unroll
        for (int m = 0; m < KPT / 4; ++m) pw[m] = *reinterpret_cast<const f32x4 *>(w + wrow(m) * K + wcol(m));
#pragma unroll
        for (int m = 0; m < APT / 4; ++m) pa[m] = *reinterpret_cast<const f32x4 *>(attn + krow(m) * C + acol(m));
#pragma unroll
        for (int m = 0; m < DPT; ++m) {
            const int e = tid + NT * m, t = min(e / NCOL, L - 1), jj = e % NCOL;
            pd[m] = Elem<T>::load_raw(a.dout, (tc + t) * rowV + h * V + j0 + jj);
        }
        pg = a.g[(tc + min(tid, L - 1)) * H + h];
        pL = L;
    };
    if (nch > 0) fetch(nch - 1);
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t ch = (sp.chunk0 + c) * H + h;
        if (!a.carry)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.dhs[ch * KV + (int64_t)(row0 + e) * V + j0 + li] = dacc[e];
        *reinterpret_cast<f32x4 *>(&dhT[li * LDK + row0]) = dacc;
#pragma unroll
        for (int m = 0; m < KPT / 8; ++m) {
            const int r = krow(m), i0 = kcol(m);
            const bool ok = r < pL;
            f32x4 k0, k1;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                k0[j] = ok ? pk[m].at(j) : 0.f;
                k1[j] = ok ? pk[m].at(4 + j) : 0.f;
            }
            *reinterpret_cast<f32x4 *>(&sk[r * LDK + i0]) = k0;
            *reinterpret_cast<f32x4 *>(&sk[r * LDK + i0 + 4]) = k1;
#pragma unroll
            for (int j = 0; j < 8; ++j) qT[(i0 + j) * LDC + r] = ok ? pq[m].at(j) : 0.f;
        }
#pragma unroll
        for (int m = 0; m < KPT / 4; ++m) {
            const int r = wrow(m), i0 = wcol(m);
#pragma unroll
            for (int j = 0; j < 4; ++j) wT[(i0 + j) * LDC + r] = pw[m][j];
        }
#pragma unroll
        for (int m = 0; m < APT / 4; ++m) {
            const int t = krow(m), s0 = acol(m);
#pragma unroll
            for (int j = 0; j < 4; ++j) aT[(s0 + j) * LDC + t] = pa[m][j];
        }
#pragma unroll
        for (int m = 0; m < DPT; ++m) {
            const int e = tid + NT * m;
            doT[(e % NCOL) * LDC + e / NCOL] = e < C * NCOL && e / NCOL < pL ? Elem<T>::from_raw(pd[m]) : 0.f;
        }
        if (tid < 64) chunk_decay<C>(tid < C && tid < pL ? pg : 0.f, sG, sEg, sEk);
        __syncthreads();
        if (c > 0) fetch(c - 1);
        if (wv < 4) {
            // ddelta rows 16 wv ..: attn^T do + exp(G_C - G_r) k dh
            f32x4 acc1 = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 aa = lds4(&aT[(16 * wv + li) * LDC + 4 * (4 * q + lg)]);
                const f32x4 bb = lds4(&doT[li * LDC + 4 * (4 * q + lg)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[e], bb[e], acc1, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f32x4 ka = lds4(&sk[(16 * wv + li) * LDK + 4 * (4 * q + lg)]);
                const f32x4 hb = lds4(&dhT[li * LDK + 4 * (4 * q + lg)]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[e], hb[e], acc2, 0, 0, 0);
            }
            float *dd = a.dd + ch * C * V;
            f32x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v4[e] = fmaf(sEk[row0 + e], acc2[e], acc1[e]);
                if (!a.carry) dd[(row0 + e) * V + j0 + li] = v4[e];
            }
            *reinterpret_cast<f32x4 *>(&ddT[li * LDC + row0]) = v4;
        } else {
            for (int e = tid - 256; e < NCOL * C; e += 256) {
                const int jj = e / C, t = e % C;
                doGT[jj * LDC + t] = sEg[t] * doT[jj * LDC + t];
            }
        }
        __syncthreads();
        // dh <- gamma dh + q^T (exp(G) do) - w^T ddelta
        dacc *= sEg[C - 1];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kk = 4 * (4 * q + lg);
            const f32x4 qa = lds4(&qT[(16 * wv + li) * LDC + kk]);
            const f32x4 ob = lds4(&doGT[li * LDC + kk]);
            const f32x4 wa = lds4(&wT[(16 * wv + li) * LDC + kk]);
            const f32x4 db = lds4(&ddT[li * LDC + kk]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[e], ob[e], dacc, 0, 0, 0);
                dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(-wa[e], db[e], dacc, 0, 0, 0);
            }
        }
        __syncthreads();
    }
    float *out = a.carry ? a.E + (cp.slot * H + h) * KV
                         : (a.dh0 && cp.first ? a.dh0 + ((int64_t)cp.seq * H + h) * KV : nullptr);
    if (out) {
#pragma unroll
        for (int e = 0; e < 4; ++e) out[(int64_t)(row0 + e) * V + j0 + li] = dacc[e];
    }
}

// ---------------------------------------------------------------- 4. grads
template <typename T, int K, int V, int C, int NT>
__global__ __launch_bounds__(NT) void bwd_grads_kernel(BwdArgs a) {
    constexpr int VP = V + 1, CP = C + 1;
    static_assert((C * C) % NT == 0 && (C * K) % NT == 0 && (C * V) % NT == 0 &&
                  (K * C) % NT == 0 && 2 * C <= NT, "uniform trip counts (put_row needs whole waves)");
    constexpr int NW = NT / 64;
    static_assert(C * CP <= C * VP, "Z fits where delta was");
    __shared__ float bDZ[C * VP];               // delta (read by dattn), then Z = dT T^T
    __shared__ float bdD[C * VP];               // ddelta
    __shared__ float bT[C * CP];                // T
    __shared__ float bX[C * CP];                // dattn
    __shared__ float bY[C * CP];                // dT^T, then dA
    __shared__ float bW[K * CP];                // dw^T
    float *const bD = bDZ, *const bZ = bDZ;
    __shared__ float sG[C], sEg[C], sEk[C], sb[C];
    // dG and dbeta of the chunk's rows: per-wave partial sums (sPw, sBw), the
    // extra terms of the last row (sLast), and the row and column sums of the
    // C x C terms (sRowA, sColA, sRowB)
    __shared__ float sPw[NW * C], sBw[NW * C], sLast[NW], sRowA[C], sColA[C], sRowB[C];
    const int wave = threadIdx.x >> 6;
    const int tid = threadIdx.x, H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    const ChunkLoc cl = locate_chunk(a.ct, chunk, C);
    const int L = cl.L;
    const int64_t tc = cl.tc;
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);
    const int64_t ch = chunk * H + h;
    const int64_t KV = (int64_t)K * V;
    // states: [K][V] at K = V = 128 (the matrix-core scans), else [V][K]
    const float *hsT = a.hs + ch * KV, *dhsT = a.dhs + ch * KV;
    const float *attn = a.attn + ch * C * C, *Ak = a.Ak + ch * C * C;
    const float *dws = a.d + ch * C * V;
    auto qx = [&](int r, int i) { return Elem<T>::load(a.q, (tc + r) * rowK + hk * K + i); };
    auto kx = [&](int r, int i) { return Elem<T>::load(a.k, (tc + r) * rowK + hk * K + i); };
    // dq, dk of this value head: the outputs themselves, or (grouped key heads)
    // fp32 rows [T, H, K] that a second kernel sums over each key head's group
    auto put_qk = [&](void *out, float *acc, int r, int i, float x) {
        if (acc) acc[((tc + r) * H + h) * K + i] = x;
        else Elem<T>::store(out, (tc + r) * rowK + hk * K + i, x);
    };
    auto vx = [&](int r, int j) { return Elem<T>::load(a.v, (tc + r) * rowV + h * V + j); };
    auto dox = [&](int r, int j) { return Elem<T>::load(a.dout, (tc + r) * rowV + h * V + j); };

    {
        const float *d = a.d + ch * C * V, *dd = a.dd + ch * C * V, *Tm = a.T + ch * C * C;
        for (int e = tid; e < C * V; e += NT) {
            bD[(e / V) * VP + e % V] = d[e];
            bdD[(e / V) * VP + e % V] = dd[e];
        }
        for (int e = tid; e < C * C; e += NT) bT[(e / C) * CP + e % C] = Tm[e];
        if (tid < C) {
            sb[tid] = tid < L ? a.beta[(tc + tid) * H + h] : 0.f;
        }
        for (int e = tid; e < NW * C; e += NT) {
            sPw[e] = 0.f;
            sBw[e] = 0.f;
        }
        if (tid < NW) sLast[tid] = 0.f;
    }
    load_cumdecay<C>(sG, sEg, sEk, a.g, tc, L, H, h);   // (synchronises)

    if constexpr (K == 128 && V == 128 && C == 64 && NT == 512) {
        // fp32 matrix-core tiles (layout as in the state scans)
        const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        // dattn = causal(do delta^T): 4 x 4 tiles of C x C, wave wv owns two
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = 2 * wv + u, tr = tile >> 2, tcol = tile & 3;
            const int r = 16 * tr + li, sc = 16 * tcol + li;   // A row, B column
            f32x4 acc = z4;
            for (int q = 0; q < 8; ++q) {
                const int j0q = 4 * (4 * q + lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ao = r < L ? dox(r, j0q + e) : 0.f;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ao, bD[sc * VP + j0q + e], acc, 0, 0, 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * tr + 4 * lg + e;
                bX[rr * CP + sc] = sc <= rr ? acc[e] : 0.f;
            }
        }
        // dw^T = -(h ddelta^T): 8 x 4 tiles of K x C, wave wv owns row tile wv
        {
            const int i = 16 * wv + li;   // A row
            f32x4 acc[4] = {z4, z4, z4, z4};
            for (int q = 0; q < 8; ++q) {
                const int j0q = 4 * (4 * q + lg);
                float ha[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) ha[e] = hsT[(int64_t)i * V + j0q + e];   // [K][V] at K = V = 128
#pragma unroll
                for (int tcol = 0; tcol < 4; ++tcol) {
                    const int rc = 16 * tcol + li;   // B column
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[tcol] = __builtin_amdgcn_mfma_f32_16x16x4f32(ha[e], bdD[rc * VP + j0q + e], acc[tcol], 0, 0, 0);
                }
            }
#pragma unroll
            for (int tcol = 0; tcol < 4; ++tcol)
#pragma unroll
                for (int e = 0; e < 4; ++e) bW[(16 * wv + 4 * lg + e) * CP + 16 * tcol + li] = -acc[tcol][e];
        }
        __syncthreads();
        // dT^T[s][r] = beta_s ((V ddelta^T)[s][r] + exp(G_s) (K dw^T)[s][r]): two tiles per wave
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tile = 2 * wv + u, ts = tile >> 2, tcol = tile & 3;
            const int sr = 16 * ts + li, rc = 16 * tcol + li;   // A row, B column
            f32x4 av = z4, ak = z4;
            for (int q = 0; q < 8; ++q) {
                const int j0q = 4 * (4 * q + lg);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = sr < L;
                    av = __builtin_amdgcn_mfma_f32_16x16x4f32(ok ? vx(sr, j0q + e) : 0.f, bdD[rc * VP + j0q + e], av, 0, 0, 0);
                    ak = __builtin_amdgcn_mfma_f32_16x16x4f32(ok ? kx(sr, j0q + e) : 0.f, bW[(j0q + e) * CP + rc], ak, 0, 0, 0);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ss = 16 * ts + 4 * lg + e;
                bY[ss * CP + rc] = sb[ss] * (av[e] + sEg[ss] * ak[e]);
            }
        }
        __syncthreads();
    } else {
        // Products with register tiles: a thread owns TR rows x TW consecutive
        // columns of the output, so each operand it loads feeds several FMAs.
        // C x C outputs: tiles of CR rows x CW columns.
        constexpr int CW = C >= 64 ? 4 : 1;
        constexpr int CG = C / CW;                       // column groups of a row
        constexpr int CR = (C * C) / (NT * CW);
        static_assert(CR >= 1 && CR * CW * NT == C * C && CG <= 64, "C x C tiles");
        // dattn[r][s] = causal(do delta^T)
        {
            const int s0 = (tid % CG) * CW, r0 = (tid / CG) * CR;
            float acc[CR][CW] = {};
            for (int j = 0; j < V; ++j) {
                float y[CW], x[CR];
    #pragma unroll
                for (int n = 0; n < CW; ++n) y[n] = bD[(s0 + n) * VP + j];
    #pragma unroll
                for (int m = 0; m < CR; ++m) x[m] = r0 + m < L ? dox(r0 + m, j) : 0.f;
    #pragma unroll
                for (int m = 0; m < CR; ++m)
    #pragma unroll
                    for (int n = 0; n < CW; ++n) acc[m][n] = fmaf(x[m], y[n], acc[m][n]);
            }
    #pragma unroll
            for (int m = 0; m < CR; ++m)
    #pragma unroll
                for (int n = 0; n < CW; ++n) bX[(r0 + m) * CP + s0 + n] = s0 + n <= r0 + m ? acc[m][n] : 0.f;
        }
        // dw^T[i][r] = -(h ddelta^T)[i][r]: K x C outputs, tiles of KR rows x CW columns
        {
            constexpr int KR = (K * C) / (NT * CW);
            static_assert(KR >= 1 && KR * CW * NT == K * C, "K x C tiles");
            const int c0 = (tid % CG) * CW, i0 = (tid / CG) * KR;
            float acc[KR][CW] = {};
            for (int j = 0; j < V; ++j) {
                float y[CW], x[KR];
    #pragma unroll
                for (int n = 0; n < CW; ++n) y[n] = bdD[(c0 + n) * VP + j];
    #pragma unroll
                for (int m = 0; m < KR; ++m) x[m] = hsT[(int64_t)j * K + i0 + m];
    #pragma unroll
                for (int m = 0; m < KR; ++m)
    #pragma unroll
                    for (int n = 0; n < CW; ++n) acc[m][n] = fmaf(x[m], y[n], acc[m][n]);
            }
    #pragma unroll
            for (int m = 0; m < KR; ++m)
    #pragma unroll
                for (int n = 0; n < CW; ++n) bW[(i0 + m) * CP + c0 + n] = -acc[m][n];
        }
        __syncthreads();
        // dT^T[s][r] = beta_s ((V ddelta^T)[s][r] + exp(G_s) (K dw^T)[s][r])
        {
            const int r0 = (tid % CG) * CW, s0 = (tid / CG) * CR;
            float av[CR][CW] = {}, ak[CR][CW] = {};
            for (int j = 0; j < V; ++j) {
                float y[CW], x[CR];
    #pragma unroll
                for (int n = 0; n < CW; ++n) y[n] = bdD[(r0 + n) * VP + j];
    #pragma unroll
                for (int m = 0; m < CR; ++m) x[m] = s0 + m < L ? vx(s0 + m, j) : 0.f;
    #pragma unroll
                for (int m = 0; m < CR; ++m)
    #pragma unroll
                    for (int n = 0; n < CW; ++n) av[m][n] = fmaf(x[m], y[n], av[m][n]);
            }
            for (int i = 0; i < K; ++i) {
                float y[CW], x[CR];
    #pragma unroll
                for (int n = 0; n < CW; ++n) y[n] = bW[i * CP + r0 + n];
    #pragma unroll
                for (int m = 0; m < CR; ++m) x[m] = s0 + m < L ? kx(s0 + m, i) : 0.f;
    #pragma unroll
                for (int m = 0; m < CR; ++m)
    #pragma unroll
                    for (int n = 0; n < CW; ++n) ak[m][n] = fmaf(x[m], y[n], ak[m][n]);
            }
    #pragma unroll
            for (int m = 0; m < CR; ++m)
    #pragma unroll
                for (int n = 0; n < CW; ++n)
                    bY[(s0 + m) * CP + r0 + n] = sb[s0 + m] * (av[m][n] + sEg[s0 + m] * ak[m][n]);
        }
        __syncthreads();
    }
    // Z = dT T^T
    for (int o = tid; o < C * C; o += NT) {
        const int r = o / C, s = o % C;
        float acc = 0.f;
        for (int p = 0; p < C; ++p) acc = fmaf(bY[p * CP + r], bT[s * CP + p], acc);
        bZ[r * CP + s] = acc;
    }
    __syncthreads();
    // dA = -strict_lower(T^T Z)   (T[p][r] = 0 for p < r)
    for (int o = tid; o < C * C; o += NT) {
        const int r = o / C, s = o % C;
        float acc = 0.f;
        if (s < r)
            for (int p = r; p < C; ++p) acc = fmaf(-bT[p * CP + r], bZ[p * CP + s], acc);
        bY[r * CP + s] = acc;
    }
    __syncthreads();

    if constexpr (K == 128 && V == 128 && C == 64 && NT == 512) {
        // dv = diag(beta) T^T ddelta, dbeta += (T^T ddelta) . v: 4 x 8 tiles of C x V,
        // wave wv owns column tile wv
        const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
        const int j = 16 * wv + li;   // B column
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 acc[4] = {z4, z4, z4, z4};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int p0 = 4 * (4 * q + lg);
            float bb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bb[e] = bdD[(p0 + e) * VP + j];
#pragma unroll
            for (int tr = 0; tr < 4; ++tr)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(bT[(p0 + e) * CP + 16 * tr + li], bb[e], acc[tr], 0, 0, 0);
        }
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                float part = 0.f;
                if (r < L) {
                    Elem<T>::store(a.dv, (tc + r) * rowV + h * V + j, sb[r] * acc[tr][e]);
                    part = acc[tr][e] * vx(r, j);
                }
                put_row<16>(sBw + wave * C, r, part);
            }
    } else {
        // dv = diag(beta) T^T ddelta;  dbeta += (T^T ddelta) . v
        for (int o = tid; o < C * V; o += NT) {
            const int r = o / V, j = o % V;
            float dvb = 0.f;
            for (int p = r; p < C; ++p) dvb = fmaf(bT[p * CP + r], bdD[p * VP + j], dvb);
            float part = 0.f;
            if (r < L) {
                Elem<T>::store(a.dv, (tc + r) * rowV + h * V + j, sb[r] * dvb);
                part = dvb * vx(r, j);
            }
            put_row<V>(sBw + wave * C, r, part);
        }
    }
    // attn and A through the decay: with e = dattn attn + beta_r dA Ak (the
    // raw gradient matrices), dG_r += e(r, s) and dG_s -= e(r, s); dbeta_r += dA Ak.
    // One thread sums each row and each column, in order.
    if (tid < C) {
        const int r = tid;
        float re = 0.f, rb = 0.f;
        for (int s2 = 0; s2 <= r; ++s2) {
            const float eA = s2 < r ? bY[r * CP + s2] * Ak[r * C + s2] : 0.f;
            re += bX[r * CP + s2] * attn[r * C + s2] + sb[r] * eA;
            rb += eA;
        }
        sRowA[r] = re;
        sRowB[r] = rb;
    } else if (tid < 2 * C) {
        const int s2 = tid - C;
        float ce = 0.f;
        for (int r = s2; r < C; ++r) {
            const float eA = s2 < r ? bY[r * CP + s2] * Ak[r * C + s2] : 0.f;
            ce += bX[r * CP + s2] * attn[r * C + s2] + sb[r] * eA;
        }
        sColA[s2] = ce;
    }
    __syncthreads();
    // fold the decay in once: bX <- dattn (.) D,  bY <- dA (.) beta_r D  (= dKK)
    for (int o = tid; o < C * C; o += NT) {
        const int r = o / C, s = o % C;
        if (s <= r) {
            const float dec = expf(sG[r] - sG[s]);
            bX[r * CP + s] *= dec;
            bY[r * CP + s] *= sb[r] * dec;
        }
    }
    __syncthreads();
    if constexpr (K == 128 && C == 64 && NT == 512) {
        // dq and dk on the fp32 matrix cores: 16 x 16 output tiles, wave wv owns
        // column tile 16 wv and the four row tiles.  Operand and accumulator
        // layout as in the state scans: lane (li, lg) gives A[li][k], B[k][li]
        // with k = 4 (4 q + lg) + e, and holds D[4 lg + e][li].
        const int lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
        const int i = 16 * wv + li;
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 dqg[4], dkt[4], qa[4], dkr[4], dkb[4];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) dqg[tr] = dkt[tr] = qa[tr] = dkr[tr] = dkb[tr] = z4;
        // over V:  dqg = do h^T,  dkt = delta dh^T  (the k_tilde gradient)
        for (int q = 0; q < 8; ++q) {
            const int j0q = 4 * (4 * q + lg);
            float hb[4], dhb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hb[e] = hsT[(int64_t)i * V + j0q + e];
                dhb[e] = dhsT[(int64_t)i * V + j0q + e];
            }
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
                const int r = 16 * tr + li;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ao = r < L ? dox(r, j0q + e) : 0.f;
                    dqg[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(ao, hb[e], dqg[tr], 0, 0, 0);
                    dkt[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(dws[r * V + j0q + e], dhb[e], dkt[tr], 0, 0, 0);
                }
            }
        }
        // over the chunk's tokens p (zero past L in every B operand):
        //   qa = (dattn D) k,  dkr = (dattn D)^T q + (dKK + dKK^T) k,  dkb = T^T dw
        for (int q = 0; q < 4; ++q) {
            const int p0 = 4 * (4 * q + lg);
            float kb[4], qb[4], wb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int p = p0 + e;
                kb[e] = p < L ? kx(p, i) : 0.f;
                qb[e] = p < L ? qx(p, i) : 0.f;
                wb[e] = bW[i * CP + p];
            }
#pragma unroll
            for (int tr = 0; tr < 4; ++tr) {
                const int r = 16 * tr + li;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int p = p0 + e;
                    const float xa = bX[r * CP + p], xat = bX[p * CP + r];
                    const float xy = bY[r * CP + p] + bY[p * CP + r], xt = bT[p * CP + r];
                    qa[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, kb[e], qa[tr], 0, 0, 0);
                    dkr[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xat, qb[e], dkr[tr], 0, 0, 0);
                    dkr[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xy, kb[e], dkr[tr], 0, 0, 0);
                    dkb[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt, wb[e], dkb[tr], 0, 0, 0);
                }
            }
        }
        // lane holds rows 16 tr + 4 lg + e of column i
        float pdl = 0.f;   // this lane's part of the last row's k_tilde term
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                float pg = 0.f, pd = 0.f, pk = 0.f;
                if (r < L) {
                    const float eG = sEg[r], er = sEk[r], br = sb[r];
                    const float kri = kx(r, i), qri = qx(r, i);
                    put_qk(a.dq, a.dq_acc, r, i, eG * dqg[tr][e] + qa[tr][e]);
                    put_qk(a.dk, a.dk_acc, r, i, dkr[tr][e] + er * dkt[tr][e] + br * eG * dkb[tr][e]);
                    pg = eG * dqg[tr][e] * qri - er * dkt[tr][e] * kri + br * eG * dkb[tr][e] * kri;
                    pd = er * dkt[tr][e] * kri;
                    pk = eG * dkb[tr][e] * kri;
                }
                put_row<16>(sPw + wave * C, r, pg);
                put_row<16>(sBw + wave * C, r, pk);
                pdl += pd;
            }
        }
        put_row<64>(sLast, wave, pdl);
    } else {
        // dq and dk: C x K outputs, tiles of QR rows x QW consecutive columns
        constexpr int QW = K >= 128 ? 4 : 2;
        constexpr int QG = K / QW;                   // column groups of a row
        constexpr int QR = (C * K) / (NT * QW);
        static_assert(QR >= 1 && QR * QW * NT == C * K && QG <= 64, "C x K tiles");
        const int i0 = (tid % QG) * QW, r0 = (tid / QG) * QR;
        // over the chunk's tokens p (rows p >= L hold zeros in every factor):
        //   qa  = (dattn D) k          dkr = (dattn D)^T q + (dKK + dKK^T) k
        //   dkb = T^T dw
        float qa[QR][QW] = {}, dkr[QR][QW] = {}, dkb[QR][QW] = {};
        for (int p = 0; p < L; ++p) {
            float kp[QW], qp[QW], wp[QW];
#pragma unroll
            for (int n = 0; n < QW; ++n) {
                kp[n] = kx(p, i0 + n);
                qp[n] = qx(p, i0 + n);
                wp[n] = bW[(i0 + n) * CP + p];
            }
#pragma unroll
            for (int m = 0; m < QR; ++m) {
                const int r = r0 + m;
                const float xa = bX[r * CP + p], xat = bX[p * CP + r];
                const float xy = bY[r * CP + p] + bY[p * CP + r], xt = bT[p * CP + r];
#pragma unroll
                for (int n = 0; n < QW; ++n) {
                    qa[m][n] = fmaf(xa, kp[n], qa[m][n]);
                    dkr[m][n] = fmaf(xat, qp[n], fmaf(xy, kp[n], dkr[m][n]));
                    dkb[m][n] = fmaf(xt, wp[n], dkb[m][n]);
                }
            }
        }
        //   dqg = do h^T               dkt = delta dh^T   (the k_tilde gradient)
        float dqg[QR][QW] = {}, dkt[QR][QW] = {};
        for (int j = 0; j < V; ++j) {
            float hp[QW], dhp[QW];
#pragma unroll
            for (int n = 0; n < QW; ++n) {
                hp[n] = hsT[(int64_t)j * K + i0 + n];
                dhp[n] = dhsT[(int64_t)j * K + i0 + n];
            }
#pragma unroll
            for (int m = 0; m < QR; ++m) {
                const int r = r0 + m;
                const float xo = r < L ? dox(r, j) : 0.f, xd = dws[r * V + j];
#pragma unroll
                for (int n = 0; n < QW; ++n) {
                    dqg[m][n] = fmaf(xo, hp[n], dqg[m][n]);
                    dkt[m][n] = fmaf(xd, dhp[n], dkt[m][n]);
                }
            }
        }
        float pdl = 0.f;   // this lane's part of the last row's k_tilde term
#pragma unroll
        for (int m = 0; m < QR; ++m) {
            const int r = r0 + m;
            float pg = 0.f, pd = 0.f, pk = 0.f;
            if (r < L) {
                const float eG = sEg[r], er = sEk[r], br = sb[r];
#pragma unroll
                for (int n = 0; n < QW; ++n) {
                    const int i = i0 + n;
                    const float kri = kx(r, i), qri = qx(r, i);
                    put_qk(a.dq, a.dq_acc, r, i, eG * dqg[m][n] + qa[m][n]);
                    put_qk(a.dk, a.dk_acc, r, i, dkr[m][n] + er * dkt[m][n] + br * eG * dkb[m][n]);
                    pg += eG * dqg[m][n] * qri - er * dkt[m][n] * kri + br * eG * dkb[m][n] * kri;
                    pd += er * dkt[m][n] * kri;
                    pk += eG * dkb[m][n] * kri;
                }
            }
            put_row<QG>(sPw + wave * C, r, pg);
            put_row<QG>(sBw + wave * C, r, pk);
            pdl += pd;
        }
        put_row<64>(sLast, wave, pdl);
    }
    // gamma: dG_last += gamma <h, dh>
    {
        float x = 0.f;
#pragma unroll 4
        for (int e = tid; e < K * V; e += NT) x = fmaf(hsT[e], dhsT[e], x);
        put_row<64>(sLast, wave, sEg[C - 1] * x);
    }
    __syncthreads();
    if (tid == 0) {
        float last = 0.f;
        for (int w = 0; w < NW; ++w) last += sLast[w];
        float acc = 0.f;
        for (int r = C - 1; r >= 0; --r) {
            float dG = sRowA[r] - sColA[r], db = sRowB[r];
            for (int w = 0; w < NW; ++w) {
                dG += sPw[w * C + r];
                db += sBw[w * C + r];
            }
            if (r == C - 1) dG += last;
            acc += dG;
            if (r < L) {
                a.dg[(tc + r) * H + h] = acc;
                a.dbeta[(tc + r) * H + h] = db;
            }
        }
    }
}

// ------------------------------------------------------ 4b. grads, K = V = 128, C = 64
// The same gradients as bwd_grads_kernel (bf16 inputs), arranged so that every
// matrix-core operand comes from LDS or registers: the chunk's rows of do, k,
// v and q are staged once (16-byte loads) into regions whose earlier contents
// are dead, and h, dh (stored K x V) are fetched into registers first, so
// their latency overlaps the staging; gamma <h, dh> is summed from those
// registers.  Row and column sums and the final reverse cumulative sum run
// over many threads, each combination in a fixed order (two calls give the
// same bits).  Products are 16 x 16 fp32 matrix-core tiles as in the state
// scans: lane (li, lg) gives A[li][k] and B[k][li] with k = 4 (4 q + lg) + e,
// and holds D[4 lg + e][li].
template <typename T>
__global__ __launch_bounds__(512) void bwd_grads_mfma_kernel(BwdArgs a) {
    static_assert(sizeof(typename Elem<T>::raw_t) == 2, "k, v, q rows are staged as bf16");
    constexpr int K = 128, V = 128, C = 64, NT = 512, NW = 8;
    constexpr int VP = V + 4;   // fp32 rows of C x V tiles (16-byte aligned; 16 rows hit distinct banks)
    constexpr int CP = C + 1;   // fp32 rows of C x C tiles and of dw^T [K][CP]
    constexpr int RS = K + 4;   // bf16 rows of the staged k, v, q rows [C][RS] (8-byte aligned)
    constexpr int PS = V + 8;   // bf16 rows of the delta, ddelta planes and of do [C][PS] (16-byte aligned)
    constexpr int PF = C * PS;  // floats of two [C][PS] bf16 planes
    typedef uint16_t u16;
    // LDS regions, reused as their contents die:
    //   R1:  delta as bf16 hi, lo planes -> k rows | v rows (bf16 [C][RS] each) -> k rows | Z [C][CP]
    //   bdD: ddelta as bf16 hi, lo planes -> q rows (bf16 [C][RS])
    //   R2:  do (bf16 [C][PS]) -> dw^T [K][CP]
    __shared__ __attribute__((aligned(16))) float R1[PF];
    __shared__ __attribute__((aligned(16))) float bdD[PF];
    __shared__ __attribute__((aligned(16))) float R2[C * VP];
    __shared__ float bT[C * CP];   // T
    __shared__ float bX[C * CP];   // dattn
    __shared__ float bY[C * CP];   // dT^T, then dA
    static_assert(2 * C * RS * 2 <= PF * 4 && C * CP * 4 <= C * RS * 2 && K * CP <= C * VP &&
                      C * PS * 2 <= C * VP * 4 && 2 * C * 128 * 2 <= C * VP * 4 && (RS * 2) % 8 == 0 &&
                      (PS * 2) % 16 == 0,
                  "staged tiles fit their regions; bf16 rows keep their alignment");
    float *const bW = R2;
    u16 *const dhi = reinterpret_cast<u16 *>(R1), *const dlo = dhi + C * PS;    // delta = hi + lo
    u16 *const ddhi = reinterpret_cast<u16 *>(bdD), *const ddlo = ddhi + C * PS;  // ddelta
    u16 *const bdo = reinterpret_cast<u16 *>(R2);                                // do
    u16 *const rk = reinterpret_cast<u16 *>(R1), *const rv = rk + C * RS;
    u16 *const rq = reinterpret_cast<u16 *>(bdD);
    float *const bZ = reinterpret_cast<float *>(rv);
    __shared__ float sG[C], sEg[C], sEk[C], sb[C];
    __shared__ float sPw[NW * C], sBw[NW * C], sLast[NW], sRowA[C], sColA[C], sRowB[C];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, li = lane & 15, lg = lane >> 4;
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    const ChunkLoc cl = locate_chunk(a.ct, chunk, C);
    const int L = cl.L;
    const int64_t tc = cl.tc;
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);
    const int64_t ch = chunk * H + h;
    const int64_t KV = (int64_t)K * V;
    const float *hs = a.hs + ch * KV, *dhs = a.dhs + ch * KV;   // [K][V]
    const float *attn = a.attn + ch * C * C, *Ak = a.Ak + ch * C * C;
    const int i = 16 * wv + li;   // this lane's column of the K-wide outputs (dq, dk, dw^T rows)
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    auto put_qk = [&](void *out, float *acc, int r, int ii, float x) {
        if (acc) acc[((tc + r) * H + h) * K + ii] = x;
        else Elem<T>::store(out, (tc + r) * rowK + hk * K + ii, x);
    };
    // 8 consecutive bf16 of row r (clamped into the chunk) of a [T, H, D] tensor
    auto row8 = [&](const void *base, int64_t row_elems, int64_t col0, int r) {
        const int64_t e = (tc + min(r, L - 1)) * row_elems + col0;
        return *reinterpret_cast<const uint4 *>(static_cast<const u16 *>(base) + e);
    };
    auto f32of = [](uint32_t w, int half) { return __uint_as_float(half ? (w & 0xffff0000u) : (w << 16)); };
    auto bf = [](u16 x) { return __uint_as_float((uint32_t)x << 16); };
    // x[4 tr + e] is this lane's term of row 16 tr + 4 lg + e; the sum over the
    // 16 lanes li of its lane group comes back in lane li for row index li
    // (a transposing butterfly: 15 exchanges instead of 16 x 4)
    auto rows16 = [&](float (&x)[16]) {
        float y8[8], y4[4], y2[2];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const bool hi = li & 8;
            const float send = hi ? x[t] : x[8 + t];
            y8[t] = (hi ? x[8 + t] : x[t]) + __shfl_xor(send, 8);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool hi = li & 4;
            const float send = hi ? y8[t] : y8[4 + t];
            y4[t] = (hi ? y8[4 + t] : y8[t]) + __shfl_xor(send, 4);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bool hi = li & 2;
            const float send = hi ? y4[t] : y4[2 + t];
            y2[t] = (hi ? y4[2 + t] : y4[t]) + __shfl_xor(send, 2);
        }
        const bool hi = li & 1;
        const float send = hi ? y2[0] : y2[1];
        return (hi ? y2[1] : y2[0]) + __shfl_xor(send, 1);
    };
    const int rrow = 16 * (li >> 2) + 4 * lg + (li & 3);   // the row whose sum lane li receives
    // a C x 128 bf16 tile of this chunk's rows, staged in LDS (row stride 128)
    // and written as whole rows, 16 bytes per lane
    auto write_rows = [&](const u16 *tile, void *out, int64_t row_elems, int64_t col0) {
#pragma unroll
        for (int m = 0; m < (C * 128 / 8) / NT; ++m) {
            const int e8 = tid + NT * m, r = e8 >> 4, c8 = 8 * (e8 & 15);
            if (r < L)
                *reinterpret_cast<uint4 *>(static_cast<u16 *>(out) + (tc + r) * row_elems + col0 + c8) =
                    *reinterpret_cast<const uint4 *>(&tile[r * 128 + c8]);
        }
    };

    // An fp32 operand x enters a bf16 matrix-core product as the pair hi = bf16(x),
    // lo = bf16(x - hi), |x - hi - lo| <= 2^-18 |x|: products of two such operands
    // take hi.hi + hi.lo + lo.hi, those with an exact bf16 input (do) hi + lo;
    // every product of bf16 values is exact in fp32 and the sums run in fp32.
    auto split2 = [](float x0, float x1, uint32_t &hi, uint32_t &lo) {
        hi = mfma::cvt2(x0, x1);
        lo = mfma::cvt2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
    };
    // ---- h and dh of this lane's row i, columns 32 kb + 8 lg .. + 7 (the B
    // operands of dqg, dk~ and the A operand of dw^T), fetched first, split
    // into hi, lo pairs; gamma <h, dh> summed from them (the lanes cover
    // every element once)
    mfma::bf16x8 hhi[4], hlo[4], dhhi[4], dhlo[4];
    float gam = 0.f;
    {
        f32x4 hv[8], dhv[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int64_t o = (int64_t)i * V + 32 * (m >> 1) + 8 * lg + 4 * (m & 1);
            hv[m] = *reinterpret_cast<const f32x4 *>(hs + o);
            dhv[m] = *reinterpret_cast<const f32x4 *>(dhs + o);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            uint32_t a0[4], a1[4], b0[4], b1[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x4 &x = hv[2 * kb + (t >> 1)], &y = dhv[2 * kb + (t >> 1)];
                const int e = 2 * (t & 1);
                gam = fmaf(x[e], y[e], fmaf(x[e + 1], y[e + 1], gam));
                split2(x[e], x[e + 1], a0[t], a1[t]);
                split2(y[e], y[e + 1], b0[t], b1[t]);
            }
            hhi[kb] = mfma::as8(make_uint4(a0[0], a0[1], a0[2], a0[3]));
            hlo[kb] = mfma::as8(make_uint4(a1[0], a1[1], a1[2], a1[3]));
            dhhi[kb] = mfma::as8(make_uint4(b0[0], b0[1], b0[2], b0[3]));
            dhlo[kb] = mfma::as8(make_uint4(b1[0], b1[1], b1[2], b1[3]));
        }
    }
    // ---- staging: delta and ddelta (fp32 workspace) as hi, lo planes, T, do
    // (rows past L zero), beta, decay
    {
        const float *d = a.d + ch * C * V, *dd = a.dd + ch * C * V, *Tm = a.T + ch * C * C;
#pragma unroll
        for (int m = 0; m < (C * V / 4) / NT; ++m) {
            const int e4 = tid + NT * m, r = (4 * e4) / V, j = (4 * e4) % V;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(d + 4 * e4);
            const f32x4 y = *reinterpret_cast<const f32x4 *>(dd + 4 * e4);
            uint32_t h0, h1, l0, l1;
            split2(x[0], x[1], h0, l0);
            split2(x[2], x[3], h1, l1);
            *reinterpret_cast<uint2 *>(&dhi[r * PS + j]) = make_uint2(h0, h1);
            *reinterpret_cast<uint2 *>(&dlo[r * PS + j]) = make_uint2(l0, l1);
            split2(y[0], y[1], h0, l0);
            split2(y[2], y[3], h1, l1);
            *reinterpret_cast<uint2 *>(&ddhi[r * PS + j]) = make_uint2(h0, h1);
            *reinterpret_cast<uint2 *>(&ddlo[r * PS + j]) = make_uint2(l0, l1);
        }
#pragma unroll
        for (int m = 0; m < (C * C / 4) / NT; ++m) {
            const int e4 = tid + NT * m, r = (4 * e4) / C, c0 = (4 * e4) % C;
            const f32x4 t = *reinterpret_cast<const f32x4 *>(Tm + 4 * e4);
#pragma unroll
            for (int e = 0; e < 4; ++e) bT[r * CP + c0 + e] = t[e];
        }
#pragma unroll
        for (int m = 0; m < (C * V / 8) / NT; ++m) {
            const int e8 = tid + NT * m, r = (8 * e8) / V, j = (8 * e8) % V;
            const uint4 w = row8(a.dout, rowV, h * V + j, r);
            *reinterpret_cast<uint4 *>(&bdo[r * PS + j]) = r < L ? w : make_uint4(0, 0, 0, 0);
        }
        if (tid < C) sb[tid] = tid < L ? a.beta[(tc + tid) * H + h] : 0.f;
        for (int e = tid; e < NW * C; e += NT) {
            sPw[e] = 0.f;
            sBw[e] = 0.f;
        }
        if (tid < NW) sLast[tid] = 0.f;
    }
    load_cumdecay<C>(sG, sEg, sEk, a.g, tc, L, H, h);   // (synchronises)

    // ---- dattn = causal(do delta^T): 4 x 4 tiles of C x C, wave wv owns two
    auto ld8 = [](const u16 *p) { return mfma::as8(*reinterpret_cast<const uint4 *>(p)); };
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = 2 * wv + u, tr = tile >> 2, tcol = tile & 3;
        const int r = 16 * tr + li, sc = 16 * tcol + li;   // A row, B column
        f32x4 acc = z4;
#pragma unroll
        for (int kb = 0; kb < V / 32; ++kb) {
            const int j0 = 32 * kb + 8 * lg;
            const mfma::bf16x8 ao = ld8(&bdo[r * PS + j0]);
            acc = mfma::mma32(ao, ld8(&dhi[sc * PS + j0]), acc);
            acc = mfma::mma32(ao, ld8(&dlo[sc * PS + j0]), acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int rr = 16 * tr + 4 * lg + e;
            bX[rr * CP + sc] = sc <= rr ? acc[e] : 0.f;
        }
    }
    // ---- over V: dqg = do h^T, dkt = delta dh^T (the k_tilde gradient), and
    // dw^T = -(h ddelta^T) for this wave's row tile of dw^T (row i of h)
    f32x4 dqg[4], dkt[4], dwa[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dqg[t] = dkt[t] = dwa[t] = z4;
#pragma unroll
    for (int kb = 0; kb < V / 32; ++kb) {
        const int j0 = 32 * kb + 8 * lg;
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + li;
            const mfma::bf16x8 ao = ld8(&bdo[r * PS + j0]);
            const mfma::bf16x8 ah = ld8(&dhi[r * PS + j0]), al = ld8(&dlo[r * PS + j0]);
            const mfma::bf16x8 bh = ld8(&ddhi[r * PS + j0]), bl = ld8(&ddlo[r * PS + j0]);
            dqg[tr] = mfma::mma32(ao, hhi[kb], dqg[tr]);
            dqg[tr] = mfma::mma32(ao, hlo[kb], dqg[tr]);
            dkt[tr] = mfma::mma32(ah, dhhi[kb], dkt[tr]);
            dkt[tr] = mfma::mma32(ah, dhlo[kb], dkt[tr]);
            dkt[tr] = mfma::mma32(al, dhhi[kb], dkt[tr]);
            dwa[tr] = mfma::mma32(hhi[kb], bh, dwa[tr]);
            dwa[tr] = mfma::mma32(hhi[kb], bl, dwa[tr]);
            dwa[tr] = mfma::mma32(hlo[kb], bh, dwa[tr]);
        }
    }
    // gamma: dG_last += gamma <h, dh>
    put_row<64>(sLast, wv, sEg[C - 1] * gam);
    // q rows, fetched now for the q row tile staged after dT
    uint4 pq[(C * K / 8) / NT];
#pragma unroll
    for (int m = 0; m < (C * K / 8) / NT; ++m) {
        const int e8 = tid + NT * m, r = (8 * e8) / K, j = (8 * e8) % K;
        pq[m] = row8(a.q, rowK, hk * K + j, r);
    }
    __syncthreads();
    // ---- dw^T into R2 (do is dead); k, v rows into R1 (delta is dead)
#pragma unroll
    for (int tcol = 0; tcol < 4; ++tcol)
#pragma unroll
        for (int e = 0; e < 4; ++e) bW[(16 * wv + 4 * lg + e) * CP + 16 * tcol + li] = -dwa[tcol][e];
#pragma unroll
    for (int m = 0; m < (C * K / 8) / NT; ++m) {
        const int e8 = tid + NT * m, r = (8 * e8) / K, j = (8 * e8) % K;
        uint4 wk = row8(a.k, rowK, hk * K + j, r), wvv = row8(a.v, rowV, h * V + j, r);
        if (r >= L) wk = wvv = make_uint4(0, 0, 0, 0);
        // 8-byte stores: a row of RS bf16 is 8-byte but not 16-byte aligned
        uint2 *pk = reinterpret_cast<uint2 *>(&rk[r * RS + j]), *pv = reinterpret_cast<uint2 *>(&rv[r * RS + j]);
        pk[0] = make_uint2(wk.x, wk.y);
        pk[1] = make_uint2(wk.z, wk.w);
        pv[0] = make_uint2(wvv.x, wvv.y);
        pv[1] = make_uint2(wvv.z, wvv.w);
    }
    __syncthreads();
    // ---- dT^T[s][r] = beta_s ((V ddelta^T)[s][r] + exp(G_s) (K dw^T)[s][r]): two tiles per wave
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = 2 * wv + u, ts = tile >> 2, tcol = tile & 3;
        const int sr = 16 * ts + li, rc = 16 * tcol + li;   // A row, B column
        f32x4 av = z4, ak = z4;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int j0q = 4 * (4 * q + lg);
            const uint2 v2 = *reinterpret_cast<const uint2 *>(&rv[sr * RS + j0q]);
            const uint2 k2 = *reinterpret_cast<const uint2 *>(&rk[sr * RS + j0q]);
            const float v4[4] = {f32of(v2.x, 0), f32of(v2.x, 1), f32of(v2.y, 0), f32of(v2.y, 1)};
            const float k4[4] = {f32of(k2.x, 0), f32of(k2.x, 1), f32of(k2.y, 0), f32of(k2.y, 1)};
            const uint2 dh2 = *reinterpret_cast<const uint2 *>(&ddhi[rc * PS + j0q]);
            const uint2 dl2 = *reinterpret_cast<const uint2 *>(&ddlo[rc * PS + j0q]);
            const float db[4] = {f32of(dh2.x, 0) + f32of(dl2.x, 0), f32of(dh2.x, 1) + f32of(dl2.x, 1),
                                 f32of(dh2.y, 0) + f32of(dl2.y, 0), f32of(dh2.y, 1) + f32of(dl2.y, 1)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                av = __builtin_amdgcn_mfma_f32_16x16x4f32(v4[e], db[e], av, 0, 0, 0);
                ak = __builtin_amdgcn_mfma_f32_16x16x4f32(k4[e], bW[(j0q + e) * CP + rc], ak, 0, 0, 0);
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ss = 16 * ts + 4 * lg + e;
            bY[ss * CP + rc] = sb[ss] * (av[e] + sEg[ss] * ak[e]);
        }
    }
    f32x4 dvk[4];   // dv rows 16 tr + 4 lg + e of column 16 wv + li, stored once a tile is free
    {
        // dv = diag(beta) T^T ddelta, dbeta += (T^T ddelta) . v: 4 x 8 tiles of C x V,
        // wave wv owns column tile wv (v read from its staged rows)
        const int j = 16 * wv + li;   // B column
        f32x4 acc[4] = {z4, z4, z4, z4};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int p0 = 4 * (4 * q + lg);
            float bb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bb[e] = bf(ddhi[(p0 + e) * PS + j]) + bf(ddlo[(p0 + e) * PS + j]);
#pragma unroll
            for (int tr = 0; tr < 4; ++tr)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(bT[(p0 + e) * CP + 16 * tr + li], bb[e], acc[tr], 0, 0, 0);
        }
        float part[16];
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                part[4 * tr + e] = r < L ? acc[tr][e] * bf(rv[r * RS + j]) : 0.f;
                dvk[tr][e] = sb[r] * acc[tr][e];
            }
        sBw[wv * C + rrow] = rows16(part);   // (the first write of this slot)
    }
    __syncthreads();
    // ---- Z = dT T^T (over the dead v rows), two of the 4 x 4 tiles per wave:
    // A[r][p] = dT[r][p] = bY[p][r], B[p][s] = T[s][p]; q rows into bdD (ddelta is dead)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = 2 * wv + u, tr = tile >> 2, tcol = tile & 3;
        f32x4 acc = z4;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pp = 4 * (4 * q + lg) + e;
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bY[pp * CP + 16 * tr + li], bT[(16 * tcol + li) * CP + pp],
                                                           acc, 0, 0, 0);
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) bZ[(16 * tr + 4 * lg + e) * CP + 16 * tcol + li] = acc[e];
    }
#pragma unroll
    for (int m = 0; m < (C * K / 8) / NT; ++m) {
        const int e8 = tid + NT * m, r = (8 * e8) / K, j = (8 * e8) % K;
        const uint4 w = r < L ? pq[m] : make_uint4(0, 0, 0, 0);
        uint2 *p2 = reinterpret_cast<uint2 *>(&rq[r * RS + j]);
        p2[0] = make_uint2(w.x, w.y);
        p2[1] = make_uint2(w.z, w.w);
    }
    // attn and Ak for the row and column sums, fetched before dA
    const int rr = tid >> 3, seg = tid & 7;
    float at_r[8], ak_r[8], at_c[8], ak_c[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int c8 = 8 * seg + m;
        at_r[m] = attn[rr * C + c8];
        ak_r[m] = Ak[rr * C + c8];
        at_c[m] = attn[c8 * C + rr];
        ak_c[m] = Ak[c8 * C + rr];
    }
    __syncthreads();
    // ---- dA = -strict_lower(T^T Z), two tiles per wave (those above the
    // diagonal are zero): A[r][p] = T[p][r] (zero for p < r), B[p][s] = Z[p][s]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = 2 * wv + u, tr = tile >> 2, tcol = tile & 3;
        f32x4 acc = z4;
        if (tcol <= tr) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pp = 4 * (4 * q + lg) + e;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bT[pp * CP + 16 * tr + li], bZ[pp * CP + 16 * tcol + li],
                                                               acc, 0, 0, 0);
                }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * tr + 4 * lg + e, s2 = 16 * tcol + li;
            bY[r * CP + s2] = s2 < r ? -acc[e] : 0.f;
        }
    }
    __syncthreads();
    // dv into the dead Z tile (the v rows' region), written out after the next barrier
#pragma unroll
    for (int tr = 0; tr < 4; ++tr)
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[(16 * tr + 4 * lg + e) * 128 + 16 * wv + li] = f32_to_bf16(dvk[tr][e]);
    {
        // e(r, s) = dattn attn + beta_r dA Ak (the raw gradient matrices):
        // dG_r += e(r, s), dG_s -= e(r, s), dbeta_r += dA Ak.  Thread t sums
        // eight columns of row t / 8 and eight rows of column t / 8; the eight
        // partial sums of a row (column) are combined in a fixed order.
        float re = 0.f, rb = 0.f, ce = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int s2 = 8 * seg + m;   // columns of row rr
            if (s2 <= rr) {
                const float eA = s2 < rr ? bY[rr * CP + s2] * ak_r[m] : 0.f;
                re += bX[rr * CP + s2] * at_r[m] + sb[rr] * eA;
                rb += eA;
            }
            const int r2 = 8 * seg + m;   // rows of column rr
            if (r2 >= rr) {
                const float eA = rr < r2 ? bY[r2 * CP + rr] * ak_c[m] : 0.f;
                ce += bX[r2 * CP + rr] * at_c[m] + sb[r2] * eA;
            }
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            re += __shfl_xor(re, off);
            rb += __shfl_xor(rb, off);
            ce += __shfl_xor(ce, off);
        }
        if (seg == 0) {
            sRowA[rr] = re;
            sRowB[rr] = rb;
            sColA[rr] = ce;
        }
    }
    __syncthreads();
    write_rows(rv, a.dv, rowV, (int64_t)h * V);
    // ---- fold the decay in once: bX <- dattn (.) D,  bY <- dA (.) beta_r D  (= dKK)
    for (int o = tid; o < C * C; o += NT) {
        const int r = o / C, s2 = o % C;
        if (s2 <= r) {
            const float dec = expf(sG[r] - sG[s2]);
            bX[r * CP + s2] *= dec;
            bY[r * CP + s2] *= sb[r] * dec;
        }
    }
    __syncthreads();
    // ---- over the chunk's tokens p (zero past L in every B operand):
    //   qa = (dattn D) k,  dkr = (dattn D)^T q + (dKK + dKK^T) k,  dkb = T^T dw
    // (k and q read down column i of their staged rows)
    f32x4 qa[4], dkr[4], dkb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[t] = dkr[t] = dkb[t] = z4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int p0 = 4 * (4 * q + lg);
        float kb[4], qb[4], wb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kb[e] = bf(rk[(p0 + e) * RS + i]);
            qb[e] = bf(rq[(p0 + e) * RS + i]);
            wb[e] = bW[i * CP + p0 + e];
        }
#pragma unroll
        for (int tr = 0; tr < 4; ++tr) {
            const int r = 16 * tr + li;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int pp = p0 + e;
                const float xa = bX[r * CP + pp], xat = bX[pp * CP + r];
                const float xy = bY[r * CP + pp] + bY[pp * CP + r], xt = bT[pp * CP + r];
                qa[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, kb[e], qa[tr], 0, 0, 0);
                dkr[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xat, qb[e], dkr[tr], 0, 0, 0);
                dkr[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xy, kb[e], dkr[tr], 0, 0, 0);
                dkb[tr] = __builtin_amdgcn_mfma_f32_16x16x4f32(xt, wb[e], dkb[tr], 0, 0, 0);
            }
        }
    }
    // ---- dq, dk; this lane's parts of dG, dbeta and of the last row's k_tilde term
    float pdl = 0.f, pgs[16], pks[16];
    float dqv[4][4], dkv[4][4];
#pragma unroll
    for (int tr = 0; tr < 4; ++tr) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * tr + 4 * lg + e;
            const float eG = sEg[r], er = sEk[r], br = sb[r];
            const float kri = bf(rk[r * RS + i]), qri = bf(rq[r * RS + i]);
            dqv[tr][e] = eG * dqg[tr][e] + qa[tr][e];
            dkv[tr][e] = dkr[tr][e] + er * dkt[tr][e] + br * eG * dkb[tr][e];
            const bool ok = r < L;
            pgs[4 * tr + e] = ok ? eG * dqg[tr][e] * qri - er * dkt[tr][e] * kri + br * eG * dkb[tr][e] * kri : 0.f;
            pks[4 * tr + e] = ok ? eG * dkb[tr][e] * kri : 0.f;
            pdl += ok ? er * dkt[tr][e] * kri : 0.f;
        }
    }
    sPw[wv * C + rrow] = rows16(pgs);
    sBw[wv * C + rrow] += rows16(pks);   // (this lane wrote the slot's dv term)
    put_row<64>(sLast, wv, pdl);
    if (a.dq_acc) {
        // grouped key heads: fp32 rows of every value head, summed by a later kernel
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                if (r < L) {
                    put_qk(a.dq, a.dq_acc, r, i, dqv[tr][e]);
                    put_qk(a.dk, a.dk_acc, r, i, dkv[tr][e]);
                }
            }
    }
    __syncthreads();   // (dw^T is dead: R2 takes the dq and dk rows)
    if (!a.dq_acc) {
        u16 *tq2 = reinterpret_cast<u16 *>(R2), *tk2 = tq2 + C * 128;
#pragma unroll
        for (int tr = 0; tr < 4; ++tr)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * tr + 4 * lg + e;
                tq2[r * 128 + i] = f32_to_bf16(dqv[tr][e]);
                tk2[r * 128 + i] = f32_to_bf16(dkv[tr][e]);
            }
    }
    __syncthreads();
    if (!a.dq_acc) {
        const u16 *tq2 = reinterpret_cast<const u16 *>(R2), *tk2 = tq2 + C * 128;
        write_rows(tq2, a.dq, rowK, (int64_t)hk * K);
        write_rows(tk2, a.dk, rowK, (int64_t)hk * K);
    }
    // ---- dg = reverse cumulative sum of dG over the chunk; dbeta (wave 0, lane = row)
    if (wv == 0) {
        const int r = lane;
        float dG = sRowA[r] - sColA[r], db = sRowB[r];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            dG += sPw[w * C + r];
            db += sBw[w * C + r];
        }
        if (r == C - 1) {
            float last = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) last += sLast[w];
            dG += last;
        }
        // inclusive scan from the last row down: x_r = sum_{r' >= r} dG_r'
        float x = dG;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(x, off);
            if (r + off < 64) x += y;
        }
        if (r < L) {
            a.dg[(tc + r) * H + h] = x;
            a.dbeta[(tc + r) * H + h] = db;
        }
    }
}

// ---------------------------------------------------------------- 5. grouped key heads
// A key head serves G = H / Hk value heads, so its dq, dk are the sums of
// theirs: out[t][hk][i] = sum_g acc[t][hk G + g][i].
template <typename T, int K>
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float *acc, void *out, int64_t n, int H, int Hk) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    const int G = H / Hk;
    const int i = (int)(e % K);
    const int64_t th = e / K;               // t * Hk + hk
    const float *src = acc + (th * G) * K + i;
    float x = 0.f;
    for (int g = 0; g < G; ++g) x += src[(int64_t)g * K];
    Elem<T>::store(out, e, x);
}

template <typename T, int K, int V, int C, int NCOL, int NT>
hipError_t launch_scans(const BwdArgs &a, int n_chains, const ComposeArgs *fwd, const ComposeArgs *rev,
                        hipStream_t s) {
    constexpr bool mf = K == 128 && V == 128 && C == 64 && NCOL == 16 && NT == 512;
    const int64_t units = (int64_t)n_chains * a.H;
    // (the matrix-core scans put a unit's strips on one XCD: padded grids)
    const unsigned grid = (unsigned)(mf ? strip_grid(units, V / NCOL) : units * (V / NCOL));
    const unsigned carry_grid = (unsigned)(mf ? strip_grid(units, (K + V) / NCOL) : units * ((K + V) / NCOL));
    auto states = [&](const BwdArgs &x, unsigned g) {
        if constexpr (mf)
            hipLaunchKernelGGL((bwd_states_mfma_kernel<T>), dim3(g), dim3(NT), 0, s, x);
        else
            hipLaunchKernelGGL((bwd_states_kernel<T, K, V, C, NCOL, NT>), dim3(g), dim3(NT), 0, s, x);
        return hipGetLastError();
    };
    auto dstates = [&](const BwdArgs &x, unsigned g) {
        if constexpr (mf)
            hipLaunchKernelGGL((bwd_dstates_mfma_kernel<T>), dim3(g), dim3(NT), 0, s, x);
        else
            hipLaunchKernelGGL((bwd_dstates_kernel<T, K, V, C, NCOL, NT>), dim3(g), dim3(NT), 0, s, x);
        return hipGetLastError();
    };
    hipError_t e;
    if (fwd) {
        // chains that split sequences: each chain's maps (M, U) and reverse
        // offsets E, the boundary states composed from them, then the emitting scans
        BwdArgs c = a;
        c.carry = 1;
        c.n_units = (int32_t)units;
        if ((e = states(c, carry_grid)) != hipSuccess) return e;
        if ((e = dstates(c, grid)) != hipSuccess) return e;
        if ((e = launch_compose(K, V, *fwd, s)) != hipSuccess) return e;
        if ((e = launch_compose(K, V, *rev, s)) != hipSuccess) return e;
    }
    BwdArgs x = a;
    x.carry = 0;
    x.n_units = (int32_t)units;
    if ((e = states(x, grid)) != hipSuccess) return e;
    return dstates(x, grid);
}

template <typename T, int K, int V, int C, int NCOL, int NT>
hipError_t launch_all(const BwdArgs &a, int n_chains, const ComposeArgs *fwd, const ComposeArgs *rev,
                      hipStream_t s) {
    const unsigned chunk_grid = (unsigned)(a.n_chunks * a.H);
    const unsigned chain_grid = (unsigned)((int64_t)n_chains * a.H * (V / NCOL));
    if (chunk_grid > 0) {
        if constexpr (K == 128 && V == 128 && C == 64 && NT == 512 && sizeof(typename Elem<T>::raw_t) == 2)
            hipLaunchKernelGGL((bwd_prep_mfma_kernel<T>), dim3(chunk_grid), dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_prep_kernel<T, K, V, C, NT>), dim3(chunk_grid), dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (chain_grid > 0) {
        const hipError_t e = launch_scans<T, K, V, C, NCOL, NT>(a, n_chains, fwd, rev, s);
        if (e != hipSuccess) return e;
    }
    if (chunk_grid > 0) {
        if constexpr (K == 128 && V == 128 && C == 64 && NT == 512 && sizeof(typename Elem<T>::raw_t) == 2)
            hipLaunchKernelGGL((bwd_grads_mfma_kernel<T>), dim3(chunk_grid), dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_grads_kernel<T, K, V, C, NT>), dim3(chunk_grid), dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !a.dq_acc) return e;
        const int64_t n = a.tokens * a.Hk * K;
        const unsigned grid = (unsigned)((n + 255) / 256);
        hipLaunchKernelGGL((bwd_group_sum_kernel<T, K>), dim3(grid), dim3(256), 0, s, a.dq_acc, a.dq, n, a.H, a.Hk);
        hipLaunchKernelGGL((bwd_group_sum_kernel<T, K>), dim3(grid), dim3(256), 0, s, a.dk_acc, a.dk, n, a.H, a.Hk);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_backward(int K, int V, int C, int dtype, const BwdArgs &a, int n_chains,
                           const ComposeArgs *fwd, const ComposeArgs *rev, hipStream_t s) {
    // The two state scans run one workgroup per (chain, head, 16-column strip),
    // on the fp32 matrix cores at K = V = 128.
    if (K == 128 && V == 128 && C == 64)
        return dtype == GDN_F32 ? launch_all<float, 128, 128, 64, 16, 512>(a, n_chains, fwd, rev, s)
                                : launch_all<bf16_t, 128, 128, 64, 16, 512>(a, n_chains, fwd, rev, s);
    if (K == 32 && V == 32 && C == 16)
        return dtype == GDN_F32 ? launch_all<float, 32, 32, 16, 8, 256>(a, n_chains, fwd, rev, s)
                                : launch_all<bf16_t, 32, 32, 16, 8, 256>(a, n_chains, fwd, rev, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
