// Matrix-core (MFMA) chunked scan for bf16 inputs at K = V = 128, C = 64.
//
// The computation is the chunk map of the MaxText PR "Add context
// parallelism to the Gated Delta Net" (section "Why"): per chunk of C tokens,
// with G_r the within-chunk cumulative log-decay and gamma_r = exp(G_r),
//   A[r,s] = beta_r exp(G_r - G_s) k_r.k_s (s < r),   T = (I + A)^{-1},
//   delta  = u - w h = T diag(beta) (V - diag(gamma) K h),
//   o      = diag(gamma) Q h + attn delta,   attn[r,s] = exp(G_r - G_s) q_r.k_s (s <= r),
//   h     <- gamma_C h + K^T diag(exp(G_C - G)) delta.
// (w = T diag(beta gamma) K and u = T diag(beta) V are never formed: their
// products with h are taken as T diag(beta) applied to V - diag(gamma) K h.)
// In the carrying mode the state is X = [M | h], started from [I | 0], with
// V = 0 on the M columns: the low-rank update M <- gamma M - k_tilde^T (w M)
// of section "Implementation".
//
// Layout of the work (gfx950 / CDNA4):
//  * One workgroup = 8 waves = one (chain, head) and one half of the state
//    columns: 64 value columns when emitting, the 128 M or the 128 h columns
//    when carrying.  The two halves of a (chain, head) are 8 block ids apart,
//    so round-robin dispatch puts them on one XCD and their shared q / k reads
//    meet in that XCD's L2.
//  * Waves 0-3 (consumers) own 16 (emit) or 32 (carry) state columns each,
//    kept in fp32 MFMA accumulators for the whole chain, and run the chunk
//    step for chunk j.  Waves 4-7 (producers) work ahead, so the
//    latency-bound preparation overlaps the scan; one barrier per chunk:
//      wave 4: Gram k k^T and the inverse T = (I + A)^{-1} for chunk j+1, all
//              on MFMA: diagonal 16 x 16 blocks by the product
//              (I - N)(I + N^2)(I + N^4)(I + N^8), off-diagonal blocks by block
//              recursion on T^T so that T comes out row-major, ready as the A
//              operand of T diag(beta);
//      wave 5: loads k, g, beta of chunk j+2 (issued one chunk earlier still,
//              so two chunks are in flight);
//      wave 6: loads q (one chunk ahead), writes it for the consumers, and
//              forms attn from the Gram k q^T;
//      wave 7: k^T by identity MFMAs (the operand of K^T delta) and the
//              per-row decay factors.
//  * Every LDS operand tile stores the eight k-slots a lane group feeds to a
//    16x16x32 MFMA in one 16-byte run, with the slot order chosen so that two
//    accumulator tiles (rows 0-15, 16-31) are directly the B operand of the
//    next product: the sequential path never goes through LDS.  16-byte chunks
//    are XOR-swizzled by row to keep 8-lane groups on distinct banks.
//  * Barriers wait for LDS traffic only, so register prefetches stay in flight
//    across them.
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int K = 128, V = 128, C = 64;
constexpr int NT = 512;   // 8 waves

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
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x4 to4(const f32x4 &x) {
    bf16x4 r;
    r[0] = (bf16)x[0]; r[1] = (bf16)x[1]; r[2] = (bf16)x[2]; r[3] = (bf16)x[3];
    return r;
}
// Two accumulator tiles (rows 0-15, 16-31 of a 32-row block) -> the bf16
// operand that reduces over those 32 rows.
__device__ __forceinline__ bf16x8 pack_pair(const f32x4 &lo, const f32x4 &hi) {
    bf16x8 r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
}
__device__ __forceinline__ bf16x8 join(const bf16x4 &lo, const bf16x4 &hi) {
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
}
__device__ __forceinline__ bf16x8 as8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

// Workgroup barrier that waits for this wave's LDS operations only (global
// loads issued earlier stay in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS tiles.  A row of a "wide" tile holds 128 bf16 (16 chunks of 16 B), a row
// of a "narrow" tile 64 bf16 (8 chunks).  Chunk q of row r lives at chunk
// q ^ (r & 7).  Within a 32-element block, chunk g holds the k-slots
// 8g .. 8g+7, i.e. logical elements 4g .. 4g+3 and 16+4g .. 16+4g+3.
__device__ __forceinline__ int woff(int r, int q) { return r * 256 + ((q ^ (r & 7)) << 4); }
__device__ __forceinline__ int noff(int r, int q) { return r * 128 + ((q ^ (r & 7)) << 4); }
__device__ __forceinline__ bf16x8 ldv(const bf16 *base, int byte_off) {
    return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(base) + byte_off);
}
__device__ __forceinline__ void stv(bf16 *base, int byte_off, const bf16x8 &v) {
    *reinterpret_cast<bf16x8 *>(reinterpret_cast<char *>(base) + byte_off) = v;
}

struct Lds {
    bf16 kR[3][C * K];      // k rows, wide tiles (loader writes j+2, producers read j+1, consumers j)
    bf16 qR[2][C * K];      // q rows, wide tiles
    bf16 kT[2][K * C];      // k transposed, narrow tiles
    bf16 attn[2][C * C];    // attn, narrow tiles
    bf16 tb[2][C * C];      // T diag(beta), narrow tiles
    float graw[3][C], braw[3][C];   // g, beta of the chunk (zero past its end)
    float gam[2][C];        // exp(G_r)
    float kdec[2][C];       // exp(G_C - G_r)
    float gC[2][4];         // exp(G_C)
    float p0G[C];           // scratch of wave 4
    float p2G[C];           // scratch of wave 6
};

// 16 x 32 tile of a bf16 row-major matrix in the MFMA register layout: lane
// (i, g) holds elements 32 kk + 4g .. +3 and 32 kk + 16 + 4g .. +3 of its row.
//
// Rows past the end of a ragged chunk: callers clamp the row to the last
// valid token instead of zeroing it, so every load is unconditional and stays
// in flight.  This is exact because those rows get g = 0 and beta = 0 (the
// padding of the MaxText PR, section "Implementation"): their rows of A and of
// T diag(beta), and the columns of T diag(beta), vanish, so a duplicated k, q
// or v row only ever meets a zero factor and its outputs are not stored.
__device__ __forceinline__ uint4 load_slots(const bf16 *rowp, int kk, int lg) {
    const uint2 lo = *reinterpret_cast<const uint2 *>(rowp + 32 * kk + 4 * lg);
    const uint2 hi = *reinterpret_cast<const uint2 *>(rowp + 32 * kk + 16 + 4 * lg);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_cumsum(float x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    return x;
}

template <bool EMIT>
__global__ __launch_bounds__(NT, 1) void scan_mfma_kernel(ScanArgs a, int n_units) {
    constexpr int CPW = EMIT ? 16 : 32;   // state columns per consumer wave
    constexpr int NCT = CPW / 16;
    __shared__ Lds sm;

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
    const int64_t n_chunks = (sp.t1 - sp.t0 + C - 1) / C;
    const int64_t rowK = (int64_t)H * K;   // element stride between tokens of q, k
    const int64_t rowV = (int64_t)H * V;

    const bf16 *gq = static_cast<const bf16 *>(a.q);
    const bf16 *gk = static_cast<const bf16 *>(a.k);
    const bf16 *gv = static_cast<const bf16 *>(a.v);

    auto chunk_len = [&](int64_t j) -> int {
        const int64_t rem = sp.t1 - (sp.t0 + j * C);
        return rem < C ? (int)rem : C;
    };
    auto tok = [&](int64_t j, int r) -> int64_t { return sp.t0 + j * C + r; };

    if (wv < 4) {
        // =========================== consumers ===========================
        const bool is_M = !EMIT && cg == 0;
        const int col_w = (EMIT ? 64 * cg : 0) + CPW * wv;   // first state column
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
                        X[n][t][e] = (is_M && 16 * t + 4 * lg + e == col_w + 16 * n + li) ? 1.f : 0.f;
        }
        // value rows of this wave's columns, A layout of a 16x16x16 operand:
        // lane (i, g) holds v[16 c + i][col 4g .. 4g+3]
        uint2 vA[NCT][4];
        auto load_v = [&](int64_t j) {
            if (is_M) {
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) vA[n][c] = make_uint2(0, 0);
                return;
            }
            const int L = chunk_len(j);
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int r = 16 * c + li;
                    vA[n][c] = *reinterpret_cast<const uint2 *>(
                        gv + tok(j, r < L ? r : L - 1) * rowV + h * V + col_w + 16 * n + 4 * lg);
                }
        };
        bf16x4 i16;   // identity, B operand of a 16x16x16 product
#pragma unroll
        for (int e = 0; e < 4; ++e) i16[e] = (bf16)((4 * lg + e == li) ? 1.f : 0.f);

        if (n_chunks > 0) load_v(0);
        lds_barrier();   // iteration -2: k of chunk 0 loaded
        lds_barrier();   // iteration -1: chunk 0 prepared
        for (int64_t j = 0; j < n_chunks; ++j) {
            const int b2 = (int)(j & 1), b3 = (int)(j % 3);
            const int L = chunk_len(j);
            const bf16 *kR = sm.kR[b3];
            // value tiles of this chunk in B layout, then prefetch the next chunk's
            f32x4 Vt[NCT][4];
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    Vt[n][c] = mma16(__builtin_bit_cast(bf16x4, vA[n][c]), i16, zero4());
            if (j + 1 < n_chunks) load_v(j + 1);

            bf16x8 hb[NCT][4];
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) hb[n][kk] = pack_pair(X[n][2 * kk], X[n][2 * kk + 1]);
            // Y = K X
            f32x4 Y[NCT][4];
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int c = 0; c < 4; ++c) Y[n][c] = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bf16x8 ka = ldv(kR, woff(16 * c + li, 4 * kk + lg));
#pragma unroll
                    for (int n = 0; n < NCT; ++n) Y[n][c] = mma32(ka, hb[n][kk], Y[n][c]);
                }
            // O = Q X  (scaled by gamma_r below)
            f32x4 O[4];
            if (EMIT) {
#pragma unroll
                for (int c = 0; c < 4; ++c) O[c] = zero4();
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        O[c] = mma32(ldv(sm.qR[b2], woff(16 * c + li, 4 * kk + lg)), hb[0][kk], O[c]);
            }
            // R = V - gamma (K X), packed as the operand reducing over the chunk
            const float *gam = sm.gam[b2];
            const float *kdec = sm.kdec[b2];
            bf16x8 R[NCT][2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&gam[32 * kk + 4 * lg]);
                const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&gam[32 * kk + 16 + 4 * lg]);
#pragma unroll
                for (int n = 0; n < NCT; ++n) {
                    f32x4 lo, hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[e] = Vt[n][2 * kk][e] - g0[e] * Y[n][2 * kk][e];
                        hi[e] = Vt[n][2 * kk + 1][e] - g1[e] * Y[n][2 * kk + 1][e];
                    }
                    R[n][kk] = pack_pair(lo, hi);
                }
            }
            // delta = T diag(beta) R   (T lower triangular: row tile c needs kk <= c/2)
            f32x4 D[NCT][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int n = 0; n < NCT; ++n) D[n][c] = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    if (kk <= (c >> 1)) {
                        const bf16x8 ta = ldv(sm.tb[b2], noff(16 * c + li, 4 * kk + lg));
#pragma unroll
                        for (int n = 0; n < NCT; ++n) D[n][c] = mma32(ta, R[n][kk], D[n][c]);
                    }
            }
            bf16x8 dk[NCT][2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const f32x4 k0 = *reinterpret_cast<const f32x4 *>(&kdec[32 * kk + 4 * lg]);
                const f32x4 k1 = *reinterpret_cast<const f32x4 *>(&kdec[32 * kk + 16 + 4 * lg]);
#pragma unroll
                for (int n = 0; n < NCT; ++n) {
                    f32x4 lo, hi;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[e] = k0[e] * D[n][2 * kk][e];
                        hi[e] = k1[e] * D[n][2 * kk + 1][e];
                    }
                    dk[n][kk] = pack_pair(lo, hi);
                }
            }
            if (EMIT) {
                bf16x8 db[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) db[kk] = pack_pair(D[0][2 * kk], D[0][2 * kk + 1]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const f32x4 gr = *reinterpret_cast<const f32x4 *>(&gam[16 * c + 4 * lg]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) O[c][e] *= gr[e];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        if (kk <= (c >> 1))
                            O[c] = mma32(ldv(sm.attn[b2], noff(16 * c + li, 4 * kk + lg)), db[kk], O[c]);
                }
            }
            // X = gamma_C X + K^T diag(kdec) delta
            const float gc = sm.gC[b2][0];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
#pragma unroll
                for (int n = 0; n < NCT; ++n) X[n][t] *= gc;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 ka = ldv(sm.kT[b2], noff(16 * t + li, 4 * kk + lg));
#pragma unroll
                    for (int n = 0; n < NCT; ++n) X[n][t] = mma32(ka, dk[n][kk], X[n][t]);
                }
            }
            if (EMIT) {
                bf16 *go = static_cast<bf16 *>(a.o);
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 16 * c + 4 * lg + e;
                        if (r < L) go[tok(j, r) * rowV + h * V + col_w + li] = (bf16)O[c][e];
                    }
            }
            lds_barrier();
        }
        // chain end: final state (emit, last segment) or the pair (M_r, U_r) (carry)
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
            float *dst = is_M ? a.M_out : a.U_out;
            const int ld = is_M ? K : V;
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        dst[(slot * K + 16 * t + 4 * lg + e) * ld + col_w + 16 * n + li] = X[n][t][e];
        }
        return;
    }

    // ============================ producers ============================
    // Iteration it = -2 .. n-1 (one barrier each, matching the consumers' two
    // prologue barriers and one per chunk): the loader stores chunk it+2 and
    // issues the loads of chunk it+3; waves 4, 6, 7 prepare chunk it+1.  The
    // two waves that keep loads in flight across a barrier (loader, q) run
    // their loop unrolled by two so each register set has a fixed home, and
    // always issue a load (of the last chunk when past the end).
    const int role = wv - 4;
    if (n_chunks == 0) {
        lds_barrier();
        lds_barrier();
        return;
    }
    auto clampj = [&](int64_t j) { return j < n_chunks ? j : n_chunks - 1; };
    if (role == 1) {
        // ---------------- loader: k rows, g, beta; two register sets ----------------
        uint4 kA_[4][4], kB_[4][4];
        float gA, bA, gB, bB;
        auto issue = [&](uint4 (&t)[4][4], float &gv_, float &bv_, int64_t j) {
            const int L = chunk_len(j);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = 16 * c + li;
                const bf16 *rowp = gk + tok(j, r < L ? r : L - 1) * rowK + h * K;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) t[c][kk] = load_slots(rowp, kk, lg);
            }
            const int64_t tg = tok(j, lane < L ? lane : L - 1) * H + h;
            gv_ = a.g[tg];
            bv_ = a.beta[tg];
        };
        auto store = [&](const uint4 (&t)[4][4], float gv_, float bv_, int64_t j) {
            const int b3 = (int)(j % 3);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    stv(sm.kR[b3], woff(16 * c + li, 4 * kk + lg), as8(t[c][kk]));
            sm.graw[b3][lane] = gv_;   // raw: readers zero the rows past the chunk end
            sm.braw[b3][lane] = bv_;
        };
        issue(kA_, gA, bA, 0);
        for (int64_t it = -2; it < n_chunks; it += 2) {
            issue(kB_, gB, bB, clampj(it + 3));
            if (it + 2 < n_chunks) store(kA_, gA, bA, it + 2);
            lds_barrier();
            if (it + 1 >= n_chunks) break;
            issue(kA_, gA, bA, clampj(it + 4));
            if (it + 3 < n_chunks) store(kB_, gB, bB, it + 3);
            lds_barrier();
        }
        return;
    }
    if (role == 2) {
        // -------- q rows (one chunk ahead) -> qR, and attn from the Gram k q^T --------
        if (!EMIT) {
            for (int64_t it = -2; it < n_chunks; ++it) lds_barrier();
            return;
        }
        uint4 qA_[4][4], qB_[4][4];
        auto issue = [&](uint4 (&t)[4][4], int64_t j) {
            const int L = chunk_len(j);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = 16 * c + li;
                const bf16 *rowp = gq + tok(j, r < L ? r : L - 1) * rowK + h * K;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) t[c][kk] = load_slots(rowp, kk, lg);
            }
        };
        auto work = [&](const uint4 (&qa)[4][4], int64_t jn) {
            const int b2 = (int)(jn & 1), b3 = (int)(jn % 3);
            const int L = chunk_len(jn);
            const bf16 *kR = sm.kR[b3];
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) stv(sm.qR[b2], woff(16 * c + li, 4 * kk + lg), as8(qa[c][kk]));
            const float G = wave_cumsum(lane < L ? sm.graw[b3][lane] : 0.f, lane);
            sm.p2G[lane] = G;
            // Gram block (b, a) of K Q^T: lane (j, g) element e holds
            // k_{16b+4g+e} . q_{16a+j} = raw attn[r = 16a + j][s = 16b + 4g + e]
            bf16x4 at[4][4];
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                bf16x8 kb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kb[kk] = ldv(kR, woff(16 * bb + li, 4 * kk + lg));
                const f32x4 Gs = *reinterpret_cast<const f32x4 *>(&sm.p2G[16 * bb + 4 * lg]);
#pragma unroll
                for (int aa = bb; aa < 4; ++aa) {
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) acc = mma32(kb[kk], as8(qa[aa][kk]), acc);
                    const int r = 16 * aa + li;
                    const float Gr = sm.p2G[r];
                    f32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int s = 16 * bb + 4 * lg + e;
                        v[e] = (s <= r) ? __expf(Gr - Gs[e]) * acc[e] : 0.f;
                    }
                    at[aa][bb] = to4(v);
                }
            }
            bf16x4 z4;
            z4[0] = z4[1] = z4[2] = z4[3] = (bf16)0.f;
#pragma unroll
            for (int aa = 0; aa < 4; ++aa)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    if (kk <= (aa >> 1))
                        stv(sm.attn[b2], noff(16 * aa + li, 4 * kk + lg),
                            join(at[aa][2 * kk], (2 * kk + 1 <= aa) ? at[aa][2 * kk + 1] : z4));
        };
        issue(qA_, 0);
        lds_barrier();   // iteration -2
        for (int64_t it = -1; it < n_chunks; it += 2) {
            issue(qB_, clampj(it + 2));
            if (it + 1 < n_chunks) work(qA_, it + 1);
            lds_barrier();
            if (it + 1 >= n_chunks) break;
            issue(qA_, clampj(it + 3));
            if (it + 2 < n_chunks) work(qB_, it + 2);
            lds_barrier();
        }
        return;
    }
    for (int64_t it = -2; it < n_chunks; ++it) {
        const int64_t jn = it + 1;   // chunk being prepared
        if (jn >= 0 && jn < n_chunks) {
            const int b2 = (int)(jn & 1), b3 = (int)(jn % 3);
            const bf16 *kR = sm.kR[b3];
            const int L = chunk_len(jn);
            const float G = wave_cumsum(lane < L ? sm.graw[b3][lane] : 0.f, lane);
            if (role == 3) {
                // ---- per-row factors, and k^T by identity products
                const float GC = __shfl(G, 63);
                sm.gam[b2][lane] = __expf(G);
                sm.kdec[b2][lane] = __expf(GC - G);
                if (lane == 0) sm.gC[b2][0] = __expf(GC);
                bf16 *kT = sm.kT[b2];
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    bf16x8 id;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        id[e] = (bf16)(((e >> 2) == (n & 1) && 4 * lg + (e & 3) == li) ? 1.f : 0.f);
                    f32x4 d[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        d[c] = mma32(ldv(kR, woff(16 * c + li, 4 * (n >> 1) + lg)), id, zero4());
                    // lane (j, g) of d[c] holds k[16c + 4g + e][16n + j]
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        stv(kT, noff(16 * n + li, 4 * kk + lg), pack_pair(d[2 * kk], d[2 * kk + 1]));
                }
            } else {
                // ---- role 0: A = beta_r exp(G_r - G_s) k_r . k_s and T = (I + A)^{-1}
                sm.p0G[lane] = G;
                const float *braw = sm.braw[b3];
                bf16x8 ka[4][4];
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) ka[c][kk] = ldv(kR, woff(16 * c + li, 4 * kk + lg));
                // factors at rows 16t + 4g + e (B layout rows) and 16t + j (B layout column)
                f32x4 Gr4[4], Br4[4];
                float Gc[4], Bc[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    Gr4[t] = *reinterpret_cast<const f32x4 *>(&sm.p0G[16 * t + 4 * lg]);
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&braw[16 * t + 4 * lg]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Br4[t][e] = (16 * t + 4 * lg + e < L) ? b4[e] : 0.f;
                    Gc[t] = sm.p0G[16 * t + li];
                    Bc[t] = (16 * t + li < L) ? braw[16 * t + li] : 0.f;
                }
                // Gram blocks; AB[a][b] (a > b): B layout of A_ab; NB / NA: B / A layout of A_aa
                bf16x4 AB[4][4], NB[4], NA[4];
#pragma unroll
                for (int aa = 0; aa < 4; ++aa)
#pragma unroll
                    for (int bb = 0; bb <= aa; ++bb) {
                        f32x4 acc = zero4();
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) acc = mma32(ka[aa][kk], ka[bb][kk], acc);
                        if (aa > bb) {
                            f32x4 v;
#pragma unroll
                            for (int e = 0; e < 4; ++e)   // r = 16aa+4g+e > s = 16bb+j
                                v[e] = Br4[aa][e] * __expf(Gr4[aa][e] - Gc[bb]) * acc[e];
                            AB[aa][bb] = to4(v);
                        } else {
                            f32x4 vb, va;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int x = 4 * lg + e;   // B layout row / A layout column
                                const float ex = __expf(-fabsf(Gr4[aa][e] - Gc[aa]));
                                vb[e] = (li < x) ? Br4[aa][e] * ex * acc[e] : 0.f;
                                va[e] = (x < li) ? Bc[aa] * ex * acc[e] : 0.f;
                            }
                            NB[aa] = to4(vb);
                            NA[aa] = to4(va);
                        }
                    }
                // diagonal inverses: P = B layout of T_aa, Q = A layout of T_aa
                f32x4 Pf[4], Qf[4];
                bf16x4 P[4], Q[4];
#pragma unroll
                for (int aa = 0; aa < 4; ++aa) {
                    auto plus_i = [&](const f32x4 &m) {
                        f32x4 r = m;
#pragma unroll
                        for (int e = 0; e < 4; ++e) r[e] += (4 * lg + e == li) ? 1.f : 0.f;
                        return to4(r);
                    };
                    const f32x4 n2b = mma16(NA[aa], NB[aa], zero4());
                    const f32x4 n2a = mma16(NB[aa], NA[aa], zero4());
                    const bf16x4 n2b_ = to4(n2b), n2a_ = to4(n2a);
                    const f32x4 n4b = mma16(n2a_, n2b_, zero4());
                    const f32x4 n4a = mma16(n2b_, n2a_, zero4());
                    const bf16x4 n4b_ = to4(n4b), n4a_ = to4(n4a);
                    const f32x4 n8b = mma16(n4a_, n4b_, zero4());
                    const f32x4 n8a = mma16(n4b_, n4a_, zero4());
                    const bf16x4 i2a = plus_i(n2a), i2b = plus_i(n2b);
                    const bf16x4 i4a = plus_i(n4a), i4b = plus_i(n4b);
                    const bf16x4 i8a = plus_i(n8a), i8b = plus_i(n8b);
                    f32x4 p1, q1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float id = (4 * lg + e == li) ? 1.f : 0.f;
                        p1[e] = id - (float)NB[aa][e];
                        q1[e] = id - (float)NA[aa][e];
                    }
                    f32x4 p = mma16(i2a, to4(p1), zero4());
                    p = mma16(i4a, to4(p), zero4());
                    p = mma16(i8a, to4(p), zero4());
                    f32x4 q = mma16(i2b, to4(q1), zero4());
                    q = mma16(i4b, to4(q), zero4());
                    q = mma16(i8b, to4(q), zero4());
                    Pf[aa] = p;
                    Qf[aa] = q;
                    P[aa] = to4(p);
                    Q[aa] = to4(q);
                }
                (void)Pf;
                // off-diagonal blocks of T^T (B layout) = blocks of T (A layout):
                // U_ij = -(T^T)_ii sum_{k=i+1..j} (A^T)_ik (T^T)_kj,  i < j
                f32x4 U01, U12, U23, U02, U13, U03;
                {
                    f32x4 y = mma16(AB[1][0], Q[1], zero4());
                    U01 = -mma16(P[0], to4(y), zero4());
                    y = mma16(AB[2][1], Q[2], zero4());
                    U12 = -mma16(P[1], to4(y), zero4());
                    y = mma16(AB[3][2], Q[3], zero4());
                    U23 = -mma16(P[2], to4(y), zero4());
                    y = mma16(AB[1][0], to4(U12), zero4());
                    y = mma16(AB[2][0], Q[2], y);
                    U02 = -mma16(P[0], to4(y), zero4());
                    y = mma16(AB[2][1], to4(U23), zero4());
                    y = mma16(AB[3][1], Q[3], y);
                    U13 = -mma16(P[1], to4(y), zero4());
                    y = mma16(AB[1][0], to4(U13), zero4());
                    y = mma16(AB[2][0], to4(U23), y);
                    y = mma16(AB[3][0], Q[3], y);
                    U03 = -mma16(P[0], to4(y), zero4());
                }
                // T diag(beta): in the A layout of block (rb, cb), element e of lane
                // (i, g) is column 16 cb + 4g + e -> scale by beta there.
                auto sc = [&](const f32x4 &m, int cb) {
                    f32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = m[e] * Br4[cb][e];
                    return to4(r);
                };
                bf16x4 z4;
                z4[0] = z4[1] = z4[2] = z4[3] = (bf16)0.f;
                bf16 *tb = sm.tb[b2];
                stv(tb, noff(0 + li, 0 + lg), join(sc(Qf[0], 0), z4));
                stv(tb, noff(16 + li, 0 + lg), join(sc(U01, 0), sc(Qf[1], 1)));
                stv(tb, noff(32 + li, 0 + lg), join(sc(U02, 0), sc(U12, 1)));
                stv(tb, noff(32 + li, 4 + lg), join(sc(Qf[2], 2), z4));
                stv(tb, noff(48 + li, 0 + lg), join(sc(U03, 0), sc(U13, 1)));
                stv(tb, noff(48 + li, 4 + lg), join(sc(U23, 2), sc(Qf[3], 3)));
            }
        }
        lds_barrier();
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
