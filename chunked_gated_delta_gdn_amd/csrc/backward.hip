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
// Four launches, all fp32 arithmetic on the vector ALU:
//   1. prep   (chunk, head):    T, attn, Dec (.) K K^T, w, u
//   2. states (chain, head, column group), chunks in order: the state at
//      every chunk start (stored transposed, V x K) and delta
//   3. dstates (chain, head, column group), chunks in reverse: dl/dh at every
//      chunk end (transposed) and ddelta; dh0 at the end
//   4. grads  (chunk, head):    dq, dk, dv, dg, dbeta of the chunk's tokens
// The state columns are independent under both scans (the forward's and its
// reverse), so a workgroup of 2. and 3. owns NCOL of them.
#include "dev_common.h"
#include "gdn_internal.h"

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
// and the row factors sEg[r] = exp(G_r), sEk[r] = exp(G_{C-1} - G_r).
template <int C>
__device__ __forceinline__ void load_cumdecay(float *sG, float *sEg, float *sEk, const float *g,
                                              int64_t tc, int L, int H, int h) {
    if (threadIdx.x < C) sG[threadIdx.x] = threadIdx.x < L ? g[(tc + threadIdx.x) * H + h] : 0.f;
    __syncthreads();
    if (threadIdx.x == 0) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
            acc += sG[r];
            sG[r] = acc;
        }
    }
    __syncthreads();
    if (threadIdx.x < C) {
        sEg[threadIdx.x] = expf(sG[threadIdx.x]);
        sEk[threadIdx.x] = expf(sG[C - 1] - sG[threadIdx.x]);
    }
    __syncthreads();
}

// Adds x, summed over the N consecutive lanes that share `row`, to dst[row]
// (N a power of two; every lane of the wave must call it).
template <int N>
__device__ __forceinline__ void add_row(float *dst, int row, float x) {
    constexpr int W = N < 64 ? N : 64;
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & (W - 1)) == 0) atomicAdd(&dst[row], x);
}

// ---------------------------------------------------------------- 1. prep
template <typename T, int K, int V, int C, int NT>
__global__ __launch_bounds__(NT) void bwd_prep_kernel(BwdArgs a) {
    constexpr int KP = K + 1, CP = C + 1;
    __shared__ float sk[C * KP], sq[C * KP];
    __shared__ float sA[C * CP], sT[C * CP];
    __shared__ float sG[C], sEg[C], sEk[C], sb[C], sbg[C];
    const int tid = threadIdx.x, H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    const ChunkLoc cl = locate_chunk(a.ct, chunk, C);
    const int64_t rowK = (int64_t)H * K, rowV = (int64_t)H * V;
    const int64_t ch = chunk * H + h;

    for (int e = tid; e < C * K; e += NT) {
        const int r = e / K, i = e % K;
        const bool ok = r < cl.L;
        const int64_t x = (cl.tc + r) * rowK + h * K + i;
        sk[r * KP + i] = ok ? Elem<T>::load(a.k, x) : 0.f;
        sq[r * KP + i] = ok ? Elem<T>::load(a.q, x) : 0.f;
    }
    if (tid < C) sb[tid] = tid < cl.L ? a.beta[(cl.tc + tid) * H + h] : 0.f;
    load_cumdecay<C>(sG, sEg, sEk, a.g, cl.tc, cl.L, H, h);
    if (tid < C) sbg[tid] = sb[tid] * sEg[tid];

    float *Ak = a.Ak + ch * C * C, *attn = a.attn + ch * C * C;
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
    __syncthreads();
    // T = (I + A)^{-1} by forward substitution, one column per thread
    if (tid < C) {
        const int c = tid;
        for (int r = 0; r < C; ++r) {
            float x = r == c ? 1.f : 0.f;
            if (r > c)
                for (int s = c; s < r; ++s) x = fmaf(-sA[r * CP + s], sT[s * CP + c], x);
            sT[r * CP + c] = x;
        }
    }
    __syncthreads();
    float *To = a.T + ch * C * C, *w = a.w + ch * C * K, *u = a.u + ch * C * V;
    for (int e = tid; e < C * C; e += NT) To[e] = sT[(e / C) * CP + e % C];
    for (int e = tid; e < C * K; e += NT) {
        const int r = e / K, i = e % K;
        float acc = 0.f;
        for (int s = 0; s <= r; ++s) acc = fmaf(sT[r * CP + s], sbg[s] * sk[s * KP + i], acc);
        w[e] = acc;
    }
    for (int e = tid; e < C * V; e += NT) {
        const int r = e / V, j = e % V;
        float acc = 0.f;
        for (int s = 0; s <= r && s < cl.L; ++s)
            acc = fmaf(sT[r * CP + s], sb[s] * Elem<T>::load(a.v, (cl.tc + s) * rowV + h * V + j), acc);
        u[e] = acc;
    }
}

// ---------------------------------------------------------------- 2. states
template <typename T, int K, int V, int C, int NCOL, int NT>
__global__ __launch_bounds__(NT) void bwd_states_kernel(BwdArgs a) {
    constexpr int KP = K + 1, NP = NCOL + 1, NG = V / NCOL, EPT = K * NCOL / NT;
    static_assert(V % NCOL == 0 && (K * NCOL) % NT == 0, "column groups");
    __shared__ float sw[C * KP], sk[C * KP], sh[K * NP], sd[C * NP];
    __shared__ float sG[C], sEg[C], sEk[C];
    const int tid = threadIdx.x, H = a.H;
    const int cg = blockIdx.x % NG, h = (blockIdx.x / NG) % H, n = blockIdx.x / (NG * H);
    const int j0 = cg * NCOL;
    const ChainSpan sp = chain_span(a.ct, n, C);
    const int64_t rowK = (int64_t)H * K;
    const int64_t KV = (int64_t)K * V;

    float hr[EPT];
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + NT * m, i = e % K, jj = e / K;
        hr[m] = a.h0 ? a.h0[((int64_t)n * H + h) * KV + (int64_t)i * V + j0 + jj] : 0.f;
    }
    const int64_t nch = (sp.t1 - sp.t0 + C - 1) / C;
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t tc = sp.t0 + c * C;
        const int L = (int)((sp.t1 - tc) < C ? (sp.t1 - tc) : C);
        const int64_t ch = (sp.chunk0 + c) * H + h;
        float *hs = a.hs + ch * KV;
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            hs[(int64_t)(j0 + jj) * K + i] = hr[m];
            sh[i * NP + jj] = hr[m];
        }
        load_cumdecay<C>(sG, sEg, sEk, a.g, tc, L, H, h);
        const float gamma = sEg[C - 1];
        const float *w = a.w + ch * C * K;
        for (int e = tid; e < C * K; e += NT) {
            const int r = e / K, i = e % K;
            sw[r * KP + i] = w[e];
            sk[r * KP + i] = r < L ? sEk[r] * Elem<T>::load(a.k, (tc + r) * rowK + h * K + i) : 0.f;
        }
        __syncthreads();
        const float *u = a.u + ch * C * V;
        float *d = a.d + ch * C * V;
        for (int o = tid; o < C * NCOL; o += NT) {
            const int r = o / NCOL, jj = o % NCOL;
            float acc = u[r * V + j0 + jj];
            for (int i = 0; i < K; ++i) acc = fmaf(-sw[r * KP + i], sh[i * NP + jj], acc);
            sd[r * NP + jj] = acc;
            d[r * V + j0 + jj] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            float acc = gamma * hr[m];
            for (int r = 0; r < C; ++r) acc = fmaf(sk[r * KP + i], sd[r * NP + jj], acc);
            hr[m] = acc;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- 3. dstates
template <typename T, int K, int V, int C, int NCOL, int NT>
__global__ __launch_bounds__(NT) void bwd_dstates_kernel(BwdArgs a) {
    constexpr int KP = K + 1, CP = C + 1, NP = NCOL + 1, NG = V / NCOL, EPT = K * NCOL / NT;
    static_assert(V % NCOL == 0 && (K * NCOL) % NT == 0, "column groups");
    __shared__ float sw[C * KP], sk[C * KP], sq[C * KP], sa[C * CP];
    __shared__ float sdh[K * NP], sdo[C * NP], sdd[C * NP];
    __shared__ float sG[C], sEg[C], sEk[C];
    const int tid = threadIdx.x, H = a.H;
    const int cg = blockIdx.x % NG, h = (blockIdx.x / NG) % H, n = blockIdx.x / (NG * H);
    const int j0 = cg * NCOL;
    const ChainSpan sp = chain_span(a.ct, n, C);
    const int64_t rowK = (int64_t)H * K, rowV = (int64_t)H * V;
    const int64_t KV = (int64_t)K * V;

    float dh[EPT];
#pragma unroll
    for (int m = 0; m < EPT; ++m) {
        const int e = tid + NT * m, i = e % K, jj = e / K;
        dh[m] = a.dhT ? a.dhT[((int64_t)n * H + h) * KV + (int64_t)i * V + j0 + jj] : 0.f;
    }
    const int64_t nch = (sp.t1 - sp.t0 + C - 1) / C;
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t tc = sp.t0 + c * C;
        const int L = (int)((sp.t1 - tc) < C ? (sp.t1 - tc) : C);
        const int64_t ch = (sp.chunk0 + c) * H + h;
        float *dhs = a.dhs + ch * KV;
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            dhs[(int64_t)(j0 + jj) * K + i] = dh[m];
            sdh[i * NP + jj] = dh[m];
        }
        load_cumdecay<C>(sG, sEg, sEk, a.g, tc, L, H, h);
        const float gamma = sEg[C - 1];
        const float *w = a.w + ch * C * K, *attn = a.attn + ch * C * C;
        for (int e = tid; e < C * K; e += NT) {
            const int r = e / K, i = e % K;
            const bool ok = r < L;
            const int64_t x = (tc + r) * rowK + h * K + i;
            sw[r * KP + i] = w[e];
            sk[r * KP + i] = ok ? sEk[r] * Elem<T>::load(a.k, x) : 0.f;
            sq[r * KP + i] = ok ? sEg[r] * Elem<T>::load(a.q, x) : 0.f;
        }
        for (int e = tid; e < C * C; e += NT) sa[(e / C) * CP + e % C] = attn[e];
        for (int e = tid; e < C * NCOL; e += NT) {
            const int r = e / NCOL, jj = e % NCOL;
            sdo[r * NP + jj] = r < L ? Elem<T>::load(a.dout, (tc + r) * rowV + h * V + j0 + jj) : 0.f;
        }
        __syncthreads();
        float *dd = a.dd + ch * C * V;
        for (int o = tid; o < C * NCOL; o += NT) {
            const int r = o / NCOL, jj = o % NCOL;
            float acc = 0.f;
            for (int t = r; t < C; ++t) acc = fmaf(sa[t * CP + r], sdo[t * NP + jj], acc);
            for (int i = 0; i < K; ++i) acc = fmaf(sk[r * KP + i], sdh[i * NP + jj], acc);
            sdd[r * NP + jj] = acc;
            dd[r * V + j0 + jj] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            float acc = gamma * dh[m];
            for (int r = 0; r < C; ++r) {
                acc = fmaf(sq[r * KP + i], sdo[r * NP + jj], acc);
                acc = fmaf(-sw[r * KP + i], sdd[r * NP + jj], acc);
            }
            dh[m] = acc;
        }
        __syncthreads();
    }
    if (a.dh0) {
#pragma unroll
        for (int m = 0; m < EPT; ++m) {
            const int e = tid + NT * m, i = e % K, jj = e / K;
            a.dh0[((int64_t)n * H + h) * KV + (int64_t)i * V + j0 + jj] = dh[m];
        }
    }
}

// ---------------------------------------------------------------- 4. grads
template <typename T, int K, int V, int C, int NT>
__global__ __launch_bounds__(NT) void bwd_grads_kernel(BwdArgs a) {
    constexpr int VP = V + 1, CP = C + 1;
    static_assert((C * C) % NT == 0 && (C * K) % NT == 0 && (C * V) % NT == 0 &&
                  (K * C) % NT == 0, "uniform trip counts (add_row needs whole waves)");
    static_assert(C * CP <= C * VP, "Z fits where delta was");
    __shared__ float bDZ[C * VP];               // delta (read by dattn), then Z = dT T^T
    __shared__ float bdD[C * VP];               // ddelta
    __shared__ float bT[C * CP];                // T
    __shared__ float bX[C * CP];                // dattn
    __shared__ float bY[C * CP];                // dT^T, then dA
    __shared__ float bW[K * CP];                // dw^T
    float *const bD = bDZ, *const bZ = bDZ;
    __shared__ float sG[C], sEg[C], sEk[C], sb[C], sdG[C], sdb[C];
    const int tid = threadIdx.x, H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;
    const ChunkLoc cl = locate_chunk(a.ct, chunk, C);
    const int L = cl.L;
    const int64_t tc = cl.tc;
    const int64_t rowK = (int64_t)H * K, rowV = (int64_t)H * V;
    const int64_t ch = chunk * H + h;
    const int64_t KV = (int64_t)K * V;
    const float *hsT = a.hs + ch * KV, *dhsT = a.dhs + ch * KV;   // [V][K]
    const float *attn = a.attn + ch * C * C, *Ak = a.Ak + ch * C * C;
    const float *dws = a.d + ch * C * V;
    auto qx = [&](int r, int i) { return Elem<T>::load(a.q, (tc + r) * rowK + h * K + i); };
    auto kx = [&](int r, int i) { return Elem<T>::load(a.k, (tc + r) * rowK + h * K + i); };
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
            sdG[tid] = 0.f;
            sdb[tid] = 0.f;
        }
    }
    load_cumdecay<C>(sG, sEg, sEk, a.g, tc, L, H, h);   // (synchronises)

    // dattn[r][s] = causal(do delta^T);  dw^T[i][r] = -(h ddelta^T)[i][r]
    for (int o = tid; o < C * C; o += NT) {
        const int r = o / C, s = o % C;
        float acc = 0.f;
        if (s <= r && r < L)
#pragma unroll 8
            for (int j = 0; j < V; ++j) acc = fmaf(dox(r, j), bD[s * VP + j], acc);
        bX[r * CP + s] = acc;
    }
    for (int o = tid; o < K * C; o += NT) {
        const int i = o / C, r = o % C;
        float acc = 0.f;
#pragma unroll 8
        for (int j = 0; j < V; ++j) acc = fmaf(-hsT[(int64_t)j * K + i], bdD[r * VP + j], acc);
        bW[i * CP + r] = acc;
    }
    __syncthreads();
    // dT^T[s][r] = (Vb ddelta^T)[s][r] + (Kb dw^T)[s][r]
    for (int o = tid; o < C * C; o += NT) {
        const int s = o / C, r = o % C;
        float acc = 0.f;
        if (s < L) {
            float av = 0.f, ak = 0.f;
#pragma unroll 8
            for (int j = 0; j < V; ++j) av = fmaf(vx(s, j), bdD[r * VP + j], av);
#pragma unroll 8
            for (int i = 0; i < K; ++i) ak = fmaf(kx(s, i), bW[i * CP + r], ak);
            acc = sb[s] * (av + sEg[s] * ak);
        }
        bY[s * CP + r] = acc;
    }
    __syncthreads();
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
        add_row<V>(sdb, r, part);
    }
    // attn and A through the decay: dG_r += e, dG_s -= e;  dbeta from A
    for (int o = tid; o < C * C; o += NT) {
        const int r = o / C, s = o % C;
        float ea = 0.f, eA = 0.f;
        if (s <= r) ea = bX[r * CP + s] * attn[o];
        if (s < r) eA = bY[r * CP + s] * Ak[o];
        const float e = ea + sb[r] * eA;
        if (e != 0.f) atomicAdd(&sdG[s], -e);
        add_row<C>(sdG, r, e);
        add_row<C>(sdb, r, eA);
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
    // dq and dk, one element each
    for (int o = tid; o < C * K; o += NT) {
        const int r = o / K, i = o % K;
        float pg = 0.f, pd = 0.f, pk = 0.f;
        if (r < L) {
            const float eG = sEg[r], er = sEk[r], br = sb[r];
            // q_g: dq_g = do h^T;  attn (row r): sum_s dattn[r][s] D[r][s] k_s
            float dqg = 0.f, qa = 0.f;
#pragma unroll 8
            for (int j = 0; j < V; ++j) dqg = fmaf(dox(r, j), hsT[(int64_t)j * K + i], dqg);
            for (int s = 0; s <= r; ++s) qa = fmaf(bX[r * CP + s], kx(s, i), qa);
            Elem<T>::store(a.dq, (tc + r) * rowK + h * K + i, eG * dqg + qa);
            // k as a key of attn (column r): sum_t dattn[t][r] D[t][r] q_t
            float ka = 0.f;
            for (int t = r; t < L; ++t) ka = fmaf(bX[t * CP + r], qx(t, i), ka);
            // k_tilde: dk_tilde = delta dh^T (delta from the workspace: its LDS copy is gone)
            float dkt = 0.f;
#pragma unroll 8
            for (int j = 0; j < V; ++j) dkt = fmaf(dws[r * V + j], dhsT[(int64_t)j * K + i], dkt);
            // Kb: dKb = T^T dw
            float dkb = 0.f;
            for (int p = r; p < C; ++p) dkb = fmaf(bT[p * CP + r], bW[i * CP + p], dkb);
            // A (both operands): dKK k, dKK^T k
            float kaa = 0.f;
            for (int p = 0; p < r; ++p) kaa = fmaf(bY[r * CP + p], kx(p, i), kaa);
            for (int p = r + 1; p < L; ++p) kaa = fmaf(bY[p * CP + r], kx(p, i), kaa);
            const float kri = kx(r, i);
            Elem<T>::store(a.dk, (tc + r) * rowK + h * K + i, ka + er * dkt + br * eG * dkb + kaa);
            pg = eG * dqg * qx(r, i) - er * dkt * kri + br * eG * dkb * kri;
            pd = er * dkt * kri;
            pk = eG * dkb * kri;
        }
        add_row<K>(sdG, r, pg);
        add_row<K>(sdG, C - 1, pd);
        add_row<K>(sdb, r, pk);
    }
    // gamma: dG_last += gamma <h, dh>
    {
        float x = 0.f;
#pragma unroll 4
        for (int e = tid; e < K * V; e += NT) x = fmaf(hsT[e], dhsT[e], x);
        add_row<64>(sdG, C - 1, sEg[C - 1] * x);
    }
    __syncthreads();
    if (tid == 0) {
        float acc = 0.f;
        for (int r = C - 1; r >= 0; --r) {
            acc += sdG[r];
            if (r < L) {
                a.dg[(tc + r) * H + h] = acc;
                a.dbeta[(tc + r) * H + h] = sdb[r];
            }
        }
    }
}

template <typename T, int K, int V, int C, int NCOL, int NT>
hipError_t launch_all(const BwdArgs &a, int n_chains, hipStream_t s) {
    const unsigned chunk_grid = (unsigned)(a.n_chunks * a.H);
    const unsigned chain_grid = (unsigned)((int64_t)n_chains * a.H * (V / NCOL));
    if (chunk_grid > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<T, K, V, C, NT>), dim3(chunk_grid), dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (chain_grid > 0) {
        hipLaunchKernelGGL((bwd_states_kernel<T, K, V, C, NCOL, NT>), dim3(chain_grid), dim3(NT), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_dstates_kernel<T, K, V, C, NCOL, NT>), dim3(chain_grid), dim3(NT), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (chunk_grid > 0) {
        hipLaunchKernelGGL((bwd_grads_kernel<T, K, V, C, NT>), dim3(chunk_grid), dim3(NT), 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_backward(int K, int V, int C, int dtype, const BwdArgs &a, int n_chains,
                           hipStream_t s) {
    // The two state scans run one workgroup per (chain, head, column group)
    // for the whole sequence: narrower groups when that still fits one
    // workgroup per compute unit, so that small problems fill the chip.
    if (K == 128 && V == 128 && C == 64) {
        const bool narrow = (int64_t)n_chains * a.H * (V / 8) <= 256;
        if (dtype == GDN_F32)
            return narrow ? launch_all<float, 128, 128, 64, 8, 512>(a, n_chains, s)
                          : launch_all<float, 128, 128, 64, 16, 512>(a, n_chains, s);
        return narrow ? launch_all<bf16_t, 128, 128, 64, 8, 512>(a, n_chains, s)
                      : launch_all<bf16_t, 128, 128, 64, 16, 512>(a, n_chains, s);
    }
    if (K == 32 && V == 32 && C == 16)
        return dtype == GDN_F32 ? launch_all<float, 32, 32, 16, 8, 256>(a, n_chains, s)
                                : launch_all<bf16_t, 32, 32, 16, 8, 256>(a, n_chains, s);
    return hipErrorInvalidValue;
}

}  // namespace gdn
