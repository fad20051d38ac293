// Matrix-core (MFMA) chunked scan for bf16 inputs at K = V = 128, C = 64.
//
// The computation is the chunk map of the MaxText PR "Add context
// parallelism to the Gated Delta Net" (section "Why"): per chunk of C tokens,
// with G_r the within-chunk cumulative log-decay,
//   A[r,s] = beta_r exp(G_r - G_s) k_r.k_s (s < r),  T = (I + A)^{-1},
//   w = T diag(beta exp(G)) K,  u = T diag(beta) V,
//   delta = u - w h,   o = diag(exp(G)) Q h + attn delta,
//   h <- exp(G_C) h + K^T diag(exp(G_C - G)) delta,
// with attn[r,s] = exp(G_r - G_s) q_r.k_s for s <= r.  In the carrying mode
// the state is X = [M | h] (M from I, zero h; u = 0 on the M columns), the
// low-rank update M <- gamma M - k_tilde^T (w M) of section "Implementation".
//
// Design for gfx950 (CDNA4):
//  * One workgroup = 4 waves = one (chain, head) and one half of the state
//    columns (64 value columns when emitting; the 128 M or the 128 h columns
//    when carrying).  The two halves of a (chain, head) are issued 8 block ids
//    apart so that round-robin dispatch puts them on the same XCD and their
//    shared q / k reads meet in that XCD's L2.
//  * WY preparation is recomputed inside the scan (no HBM round trip of w, u):
//    Gram matrices and the w, u products on bf16 MFMA with fp32 accumulation,
//    the 16 x 16 diagonal blocks of T = (I + A)^{-1} by fp32 forward
//    substitution (one lane per column), the off-diagonal blocks by block
//    recursion T_ij = -T_ii sum_k A_ik T_kj on bf16 MFMA.
//  * Each wave owns 16 (emit) or 32 (carry) state columns and keeps them in
//    fp32 MFMA accumulators for the whole chain.  Every 32-wide reduction
//    block of an LDS operand stores its k-slots permuted so that the
//    accumulator registers of one product (the state, delta) are directly the
//    bf16 B operand of the next: no LDS round trip on the sequential path.
//  * The next chunk's q, k, v, g, beta are prefetched into registers while the
//    current chunk is computed.
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int K = 128, V = 128, C = 64;
constexpr int NT = 256;        // threads per workgroup (4 waves)
constexpr int LDQ = K + 8;     // row stride (elements) of C x K bf16 tiles
constexpr int LDC = C + 8;     // row stride of (.) x C bf16 tiles
constexpr int LDA = C + 1;     // row stride of C x C fp32 tiles

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                       __builtin_bit_cast(short4v, b), c, 0, 0, 0);
}

// A 16x16x32 operand register holds, in lane group g (lane / 16), the eight
// k-slots 8g .. 8g+7 of a 32-wide reduction block.  Slot 8g + e stands for
// offset 16 (e / 4) + 4 g + (e % 4) of the block: exactly the rows a 16 x 16
// accumulator tile pair (rows 0-15, 16-31) gives lane group g.  perm() is the
// storage position of logical column c under that convention.
__device__ __forceinline__ int perm(int c) {
    return (c & ~31) | (((c & 15) >> 2) << 3) | (((c >> 4) & 1) << 2) | (c & 3);
}

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-bit element e (0..7) of a 16-byte vector.
__device__ __forceinline__ uint16_t half16(const uint4 &v, int e) {
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return static_cast<uint16_t>(w >> (16 * (e & 1)));
}

// Pack two accumulator tiles (rows 0-15 and 16-31 of a 32-block) into the
// bf16 B operand of a product reducing over those 32 rows.
__device__ __forceinline__ bf16x8 pack_pair(const f32x4 &lo, const f32x4 &hi) {
    bf16x8 r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
}

struct Smem {
    bf16 q[C * LDQ];       // q rows, K-slots permuted
    bf16 k[C * LDQ];       // k rows, K-slots permuted
    bf16 kT[K * LDC];      // k transposed, C-slots permuted
    bf16 vT[V * LDC];      // this workgroup's value columns, transposed, C-slots permuted
    bf16 w[C * LDQ];       // -w, K-slots permuted
    bf16 attn[C * LDC];    // attn, C-slots permuted
    bf16 tbg[C * LDC];     // T diag(beta exp(G)), C-slots permuted
    bf16 tb[C * LDC];      // T diag(beta), C-slots permuted
    float A[C * LDA];      // A (strictly lower)
    float T[C * LDA];      // T (lower, unit diagonal)
    float G[C], gam[C], kdec[C], bg[C], b[C];
    float gammaC;
};

template <bool EMIT>
__global__ __launch_bounds__(NT, 1) void scan_mfma_kernel(ScanArgs a, int n_units) {
    constexpr int CPW = EMIT ? 16 : 32;   // state columns per wave
    constexpr int NCT = CPW / 16;         // 16-column tiles per wave
    __shared__ Smem sm;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;

    const int bid = blockIdx.x;
    const int cg = (bid >> 3) & 1;
    const int unit = ((bid >> 4) << 3) | (bid & 7);
    if (unit >= n_units) return;
    const int H = a.H;
    const int h = unit % H;
    const int chain = unit / H;
    const ChainSpan sp = chain_span(a.ct, chain, C);
    const int N = a.ct.n_seqs;
    const int64_t slot = ((int64_t)sp.seg * N + sp.seq) * H + h;

    // Columns: emit -> h columns [64 cg, 64 cg + 64); carry -> M (cg 0) or h (cg 1).
    const bool has_u = EMIT || cg == 1;
    const int vcol0 = EMIT ? 64 * cg : 0;
    const int nvseg = EMIT ? 8 : (cg == 1 ? 16 : 0);   // 16-byte segments of v per row
    const int col_w = (EMIT ? 64 * cg : 0) + CPW * wv; // first state column of this wave

    const bf16 *gq = static_cast<const bf16 *>(a.q);
    const bf16 *gk = static_cast<const bf16 *>(a.k);
    const bf16 *gv = static_cast<const bf16 *>(a.v);

    // Constant zero blocks (upper triangle) of the operands read by the
    // lower-triangular products.
    for (int e = tid; e < C * LDC; e += NT) {
        sm.attn[e] = (bf16)0.f;
        sm.tbg[e] = (bf16)0.f;
        sm.tb[e] = (bf16)0.f;
    }

    // State accumulators: X[n][t] holds rows 16t + 4 lg + e of column
    // col_w + 16 n + li.
    f32x4 X[NCT][8];
    if (EMIT) {
        const float *hin = a.h_in;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                X[0][t][e] = hin ? hin[(slot * K + 16 * t + 4 * lg + e) * V + col_w + li] : 0.f;
    } else {
#pragma unroll
        for (int n = 0; n < NCT; ++n)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[n][t][e] = (cg == 0 && 16 * t + 4 * lg + e == col_w + 16 * n + li) ? 1.f : 0.f;
    }

    // Register prefetch of one chunk: 4 x 16 B of q and of k, up to 4 x 16 B of v.
    uint4 pq[4], pk[4], pv[4];
    float pg = 0.f, pb = 0.f;
    const int64_t n_chunks = (sp.t1 - sp.t0 + C - 1) / C;

    auto prefetch = [&](int64_t j) {
        const int64_t tc = sp.t0 + j * C;
        const int L = (int)((sp.t1 - tc) < C ? (sp.t1 - tc) : C);
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = tid + NT * m, row = idx >> 4, seg = idx & 15;
            const bool ok = row < L;
            const int64_t off = ((tc + row) * H + h) * (int64_t)K + 8 * seg;
            pk[m] = z;
            if (EMIT) pq[m] = z;
            if (ok) {
                pk[m] = *reinterpret_cast<const uint4 *>(gk + off);
                if (EMIT) pq[m] = *reinterpret_cast<const uint4 *>(gq + off);
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = tid + NT * m;
            pv[m] = z;
            if (nvseg && idx < 64 * nvseg) {
                const int row = idx / nvseg, seg = idx % nvseg;
                if (row < L)
                    pv[m] = *reinterpret_cast<const uint4 *>(
                        gv + ((tc + row) * H + h) * (int64_t)V + vcol0 + 8 * seg);
            }
        }
        if (tid < C) {
            const bool ok = tid < L;
            pg = ok ? a.g[(tc + tid) * H + h] : 0.f;
            pb = ok ? a.beta[(tc + tid) * H + h] : 0.f;
        }
    };

    auto store_raw = [&]() {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = tid + NT * m, row = idx >> 4, seg = idx & 15;
            const int blk = seg >> 2, mm = seg & 3;
            const int d0 = row * LDQ + 32 * blk + 16 * (mm & 1) + 4 * (mm >> 1);
            *reinterpret_cast<uint2 *>(&sm.k[d0]) = make_uint2(pk[m].x, pk[m].y);
            *reinterpret_cast<uint2 *>(&sm.k[d0 + 8]) = make_uint2(pk[m].z, pk[m].w);
            if (EMIT) {
                *reinterpret_cast<uint2 *>(&sm.q[d0]) = make_uint2(pq[m].x, pq[m].y);
                *reinterpret_cast<uint2 *>(&sm.q[d0 + 8]) = make_uint2(pq[m].z, pq[m].w);
            }
            const int pr = perm(row);
            uint16_t *kT = reinterpret_cast<uint16_t *>(sm.kT);
#pragma unroll
            for (int e = 0; e < 8; ++e) kT[(8 * seg + e) * LDC + pr] = half16(pk[m], e);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int idx = tid + NT * m;
            if (nvseg && idx < 64 * nvseg) {
                const int row = idx / nvseg, seg = idx % nvseg;
                const int pr = perm(row);
                uint16_t *vT = reinterpret_cast<uint16_t *>(sm.vT);
#pragma unroll
                for (int e = 0; e < 8; ++e) vT[(8 * seg + e) * LDC + pr] = half16(pv[m], e);
            }
        }
        if (wv == 0) {   // within-chunk cumulative log-decay and per-row factors
            float x = pg;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_up(x, d);
                if (lane >= d) x += y;
            }
            const float gc = __shfl(x, 63);
            sm.G[lane] = x;
            const float ex = __expf(x);
            sm.gam[lane] = ex;
            sm.kdec[lane] = __expf(gc - x);
            sm.b[lane] = pb;
            sm.bg[lane] = pb * ex;
            if (lane == 0) sm.gammaC = __expf(gc);
        }
    };

    if (n_chunks > 0) prefetch(0);

    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t tc = sp.t0 + j * C;
        const int L = (int)((sp.t1 - tc) < C ? (sp.t1 - tc) : C);
        __syncthreads();                       // previous chunk's readers are done
        store_raw();
        if (j + 1 < n_chunks) prefetch(j + 1);
        __syncthreads();

        // ---- Gram k k^T, lower 16 x 16 blocks -> A (fp32)
        for (int it = wv; it < 10; it += 4) {
            const int ba = it >= 6 ? 3 : it >= 3 ? 2 : it >= 1 ? 1 : 0;
            const int bb = it - ba * (ba + 1) / 2;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mma32(ld8(&sm.k[(16 * ba + li) * LDQ + 32 * kk + 8 * lg]),
                            ld8(&sm.k[(16 * bb + li) * LDQ + 32 * kk + 8 * lg]), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * ba + 4 * lg + e, s = 16 * bb + li;
                sm.A[r * LDA + s] = (s < r) ? sm.b[r] * __expf(sm.G[r] - sm.G[s]) * acc[e] : 0.f;
            }
        }
        __syncthreads();

        if (wv == 0) {
            // ---- diagonal blocks of T: lane = (block, column), fp32 forward substitution
            const int bi = lane >> 4, jc = li, o = 16 * bi;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = (r == jc) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < 15; ++s)
#pragma unroll
                for (int r = s + 1; r < 16; ++r)
                    x[r] = fmaf(-sm.A[(o + r) * LDA + o + s], x[s], x[r]);
            const float sbg = sm.bg[o + jc], sb = sm.b[o + jc];
            const int pc = perm(o + jc);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                sm.T[(o + r) * LDA + o + jc] = x[r];
                sm.tbg[(o + r) * LDC + pc] = (bf16)(x[r] * sbg);
                sm.tb[(o + r) * LDC + pc] = (bf16)(x[r] * sb);
            }
        } else if (EMIT) {
            // ---- Gram q k^T, lower blocks incl. diagonal -> attn (bf16)
            for (int it = wv - 1; it < 10; it += 3) {
                const int ba = it >= 6 ? 3 : it >= 3 ? 2 : it >= 1 ? 1 : 0;
                const int bb = it - ba * (ba + 1) / 2;
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    acc = mma32(ld8(&sm.q[(16 * ba + li) * LDQ + 32 * kk + 8 * lg]),
                                ld8(&sm.k[(16 * bb + li) * LDQ + 32 * kk + 8 * lg]), acc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * ba + 4 * lg + e, s = 16 * bb + li;
                    const float val = (s <= r) ? __expf(sm.G[r] - sm.G[s]) * acc[e] : 0.f;
                    sm.attn[r * LDC + perm(s)] = (bf16)val;
                }
            }
        }
        __syncthreads();

        // ---- off-diagonal blocks of T, by block diagonal d = 1, 2, 3
#pragma unroll
        for (int d = 1; d <= 3; ++d) {
            if (wv <= 3 - d) {
                const int bi = wv + d, bj = wv;
                f32x4 y = zero4();
                for (int bk = bj; bk < bi; ++bk) {
                    bf16x4 av, bv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        av[e] = (bf16)sm.A[(16 * bi + li) * LDA + 16 * bk + 4 * lg + e];
                        bv[e] = (bf16)sm.T[(16 * bk + 4 * lg + e) * LDA + 16 * bj + li];
                    }
                    y = mma16(av, bv, y);
                }
                bf16x4 av, bv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    av[e] = (bf16)sm.T[(16 * bi + li) * LDA + 16 * bi + 4 * lg + e];
                    bv[e] = (bf16)y[e];
                }
                const f32x4 t = mma16(av, bv, zero4());
                const int s = 16 * bj + li, ps = perm(s);
                const float sbg = sm.bg[s], sb = sm.b[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * bi + 4 * lg + e;
                    sm.T[r * LDA + s] = -t[e];
                    sm.tbg[r * LDC + ps] = (bf16)(-t[e] * sbg);
                    sm.tb[r * LDC + ps] = (bf16)(-t[e] * sb);
                }
            }
            __syncthreads();
        }

        // ---- -w = -T diag(beta exp G) K (shared) and u for this wave's columns
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
            const int n = 2 * wv + nn;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    if (kk <= (c >> 1))
                        acc = mma32(ld8(&sm.tbg[(16 * c + li) * LDC + 32 * kk + 8 * lg]),
                                    ld8(&sm.kT[(16 * n + li) * LDC + 32 * kk + 8 * lg]), acc);
                const int pc = perm(16 * n + li);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.w[(16 * c + 4 * lg + e) * LDQ + pc] = (bf16)(-acc[e]);
            }
        }
        f32x4 D[NCT][4];
#pragma unroll
        for (int n = 0; n < NCT; ++n)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f32x4 acc = zero4();
                if (has_u) {
                    const int vr = CPW * wv + 16 * n + li;   // local value column
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        if (kk <= (c >> 1))
                            acc = mma32(ld8(&sm.tb[(16 * c + li) * LDC + 32 * kk + 8 * lg]),
                                        ld8(&sm.vT[vr * LDC + 32 * kk + 8 * lg]), acc);
                }
                D[n][c] = acc;
            }
        __syncthreads();

        // ---- the chunk step: delta = u - w X ; (o = gam Q X + attn delta) ; X = gC X + K^T kdec delta
        bf16x8 xb[NCT][4];
#pragma unroll
        for (int n = 0; n < NCT; ++n)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) xb[n][kk] = pack_pair(X[n][2 * kk], X[n][2 * kk + 1]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x8 wa = ld8(&sm.w[(16 * c + li) * LDQ + 32 * kk + 8 * lg]);
#pragma unroll
                for (int n = 0; n < NCT; ++n) D[n][c] = mma32(wa, xb[n][kk], D[n][c]);
            }
        f32x4 O[4];
        if (EMIT) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                O[c] = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    O[c] = mma32(ld8(&sm.q[(16 * c + li) * LDQ + 32 * kk + 8 * lg]), xb[0][kk], O[c]);
#pragma unroll
                for (int e = 0; e < 4; ++e) O[c][e] *= sm.gam[16 * c + 4 * lg + e];
            }
        }
        bf16x8 dk[NCT][2];
#pragma unroll
        for (int n = 0; n < NCT; ++n)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                f32x4 lo = D[n][2 * kk], hi = D[n][2 * kk + 1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    lo[e] *= sm.kdec[32 * kk + 4 * lg + e];
                    hi[e] *= sm.kdec[32 * kk + 16 + 4 * lg + e];
                }
                dk[n][kk] = pack_pair(lo, hi);
            }
        if (EMIT) {
            bf16x8 db[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) db[kk] = pack_pair(D[0][2 * kk], D[0][2 * kk + 1]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    if (kk <= (c >> 1))
                        O[c] = mma32(ld8(&sm.attn[(16 * c + li) * LDC + 32 * kk + 8 * lg]), db[kk], O[c]);
        }
        const float gC = sm.gammaC;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 ka = ld8(&sm.kT[(16 * t + li) * LDC + 32 * kk + 8 * lg]);
#pragma unroll
                for (int n = 0; n < NCT; ++n) {
                    if (kk == 0) X[n][t] *= gC;
                    X[n][t] = mma32(ka, dk[n][kk], X[n][t]);
                }
            }
        }
        if (EMIT) {
            bf16 *go = static_cast<bf16 *>(a.o);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * c + 4 * lg + e;
                    if (row < L) go[((tc + row) * H + h) * (int64_t)V + col_w + li] = (bf16)O[c][e];
                }
        }
    }

    // ---- chain end: final state (emit, last segment) or the pair (M_r, U_r) (carry)
    if (EMIT) {
        if (a.h_out && sp.seg == a.ct.n_seg - 1) {
            const int64_t so = (int64_t)sp.seq * H + h;
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.h_out[(so * K + 16 * t + 4 * lg + e) * V + col_w + li] = X[0][t][e];
        }
    } else {
        float *dst = cg == 0 ? a.M_out : a.U_out;
        const int ld = cg == 0 ? K : V;
#pragma unroll
        for (int n = 0; n < NCT; ++n)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    dst[(slot * K + 16 * t + 4 * lg + e) * ld + col_w + 16 * n + li] = X[n][t][e];
    }
}

}  // namespace

bool mfma_scan_available(int K_, int V_, int C_, int dtype) {
    return K_ == K && V_ == V && C_ == C && dtype == GDN_BF16;
}

hipError_t launch_scan_mfma(int K_, int V_, int C_, int dtype, bool carry, const ScanArgs &a,
                            hipStream_t s, bool *handled) {
    *handled = false;
    if (!mfma_scan_available(K_, V_, C_, dtype) || a.wy_w != nullptr) return hipSuccess;
    *handled = true;
    const int64_t units = (int64_t)a.n_chains * a.H;
    if (units == 0) return hipSuccess;
    const int64_t grid = ((units + 7) / 8) * 16;   // two column halves, 8 ids apart
    if (carry)
        hipLaunchKernelGGL(scan_mfma_kernel<false>, dim3((unsigned)grid), dim3(NT), 0, s, a,
                           (int)units);
    else
        hipLaunchKernelGGL(scan_mfma_kernel<true>, dim3((unsigned)grid), dim3(NT), 0, s, a,
                           (int)units);
    return hipGetLastError();
}

}  // namespace gdn
