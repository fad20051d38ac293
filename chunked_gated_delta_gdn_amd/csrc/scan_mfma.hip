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
// With A = diag(beta) A0, where A0[r,s] = exp(G_r - G_s) k_r.k_s, the identity
// (I + diag(beta) A0)^{-1} diag(beta) = diag(beta) (I + A0 diag(beta))^{-1}
// moves beta off T: the kernel inverts T' = (I + A0 diag(beta))^{-1}, whose
// strictly lower part scales columns by beta, and delta = diag(beta) T' R,
// with the row factor beta folded into exp(G_C - G_r) for the state update
// and into the columns of attn for o.
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
//    step for chunk j, reading the operand fragments of a k-block (or of two
//    row tiles) while the products of the previous one run.  Each consumer
//    shares its SIMD with one producer: a lone wave per SIMD cannot hide the
//    LDS and MFMA latencies of the chunk step (two 32-column consumers, each
//    alone on a SIMD, took 7.6k cycles per chunk against 4.5k for four
//    16-column ones).  Waves 4-7 (producers) work ahead, so the
//    latency-bound preparation overlaps the scan; one barrier per chunk:
//      wave 4: the inverse T = (I + A)^{-1} for chunk j+1, all on MFMA:
//              diagonal 16 x 16 blocks by recursive doubling of the block
//              size (diag_inverse), off-diagonal blocks by block recursion on
//              T^T so that T comes out row-major, ready as the A operand of
//              T diag(beta);
//      wave 5: loads k, g, beta of chunk j+2 (issued one chunk earlier still,
//              so two chunks are in flight), stores k, the cumulative decay,
//              and, from the k rows still in its registers, the Gram k k^T
//              with the decay factors of A;
//      wave 6: loads q (one chunk ahead), writes it for the consumers, and
//              forms attn diag(beta) from the Gram k q^T;
//      wave 7: the per-row decay factors, and K^T diag(exp(G_C - G) beta) by
//              identity MFMAs (the operand of the state update).
//  * Every LDS operand tile stores the eight k-slots a lane group feeds to a
//    16x16x32 MFMA in one 16-byte run.  Where the reduction runs over the
//    tokens of a chunk (T', attn, K^T), the slot order is chosen so that two
//    accumulator tiles (rows 0-15, 16-31) are directly the B operand of the
//    next product: the sequential path never goes through LDS.  The q, k (and
//    w) row tiles keep their elements in natural order, stored as whole rows;
//    the state rows are permuted to match instead: accumulator row
//    32b + 16h + 4g + e of X holds state row 32b + 8g + 4h + e (srow),
//    so that pack_pair of accumulator tiles 2b, 2b + 1 meets k-slots
//    8g .. 8g+7 of block b in their natural order.  The permutation only shows
//    where states enter and leave (h_in, h_out, M, U).  16-byte chunks are
//    XOR-swizzled by row (xoff, noff) against LDS bank conflicts.
//  * Barriers wait for LDS traffic only, so register prefetches stay in flight
//    across them.
#include "dev_common.h"
#include "gdn_internal.h"
#include "mfma_tile.h"

namespace gdn {
namespace {
using namespace mfma;

constexpr int K = 128, V = 128, C = 64;
constexpr int NT = 512;   // 8 waves

template <bool WY> struct Lds;
// WY factors recomputed in the kernel
template <> struct Lds<false> {
    bf16 kR[3][C * K];      // k rows, wide tiles (loader writes j+2, producers read j+1, consumers j)
    bf16 qR[2][C * K];      // q rows, wide tiles
    bf16 kT[2][K * C];      // K^T diag(kdec), narrow tiles
    bf16 attn[2][C * C];    // attn, narrow tiles
    bf16 tb[2][C * C];      // T' = (I + A0 diag(beta))^{-1}, narrow tiles
    uint2 ab[2][10][64];    // loader -> wave 4, per lane 4 bf16: the 6 off-diagonal
                            // blocks of A (B layout) and the 4 raw diagonal blocks of k k^T
    float G2[2][C];         // cumulative log-decay of the chunk, times log2(e)
    float B[2][C];          // beta (zero past the chunk end)
    float gam[2][C];        // exp(G_r); gam[63] = exp(G_C)
    float kdec[2][C];       // exp(G_C - G_r) beta_r (folded into the kT tile)
    float Gb[2][C];         // G2 - log2|beta|: exp2(G2_r - Gb_s) = exp(G_r - G_s) |beta_s|
    int negb[2];            // 1 if some beta of the chunk is negative
};
// WY factors read from a workspace: w rows replace the k rows as the
// consumers' operand, there is no Gram or T'; k is read only by producers, so
// two buffers suffice
template <> struct Lds<true> {
    bf16 kR[2][C * K];      // k rows (loader writes j+2, producers read j+1)
    bf16 qR[2][C * K];      // q rows
    bf16 wR[2][C * K];      // w rows (w wave writes j+1, consumers read j)
    bf16 kT[2][K * C];      // K^T diag(kdec)
    bf16 attn[2][C * C];    // attn
    float G2[2][C];         // cumulative log2-decay
    float gam[2][C];        // exp(G_r)
    float kdec[2][C];       // exp(G_C - G_r) (folded into the kT tile)
};

// What one workgroup works on: a chain (its tokens and first chunk), a head,
// the state row of its incoming state (emitting) or of its pair (carrying),
// and whether and where it writes the final state (emitting).
struct ScanUnit {
    ChainSpan sp;
    int h;
    int64_t slot;
    int64_t out_slot;
    bool final_state;
};

__device__ __forceinline__ ScanUnit scan_unit(const UnitRef &r, int h) {
    ScanUnit u;
    u.sp = r.sp;
    u.h = h;
    u.slot = r.slot;
    u.out_slot = r.out_slot;
    u.final_state = r.final_state;
    return u;
}

// Workgroup id -> (unit, column half): the two halves of a unit are 8 ids apart,
// so that round-robin dispatch puts them on one XCD.
// State row held by element e of accumulator tile t in lane group g (see the
// layout notes above): accumulator row 16t + 4g + e is state row
// 8g + srow(t, e), srow(t, e) = 32(t / 2) + 4(t % 2) + e (a constant).
__host__ __device__ constexpr int srow(int t, int e) { return 32 * (t >> 1) + 4 * (t & 1) + e; }

__device__ __forceinline__ int unit_of_block(int bid) { return ((bid >> 4) << 3) | (bid & 7); }
__device__ __forceinline__ int half_of_block(int bid) { return (bid >> 3) & 1; }

template <bool EMIT, bool WY, bool PACKED>
__device__ __forceinline__ void scan_body(Lds<WY> &sm, const ScanArgs &a, const ScanUnit &u, int cg) {
    constexpr int CPW = EMIT ? 16 : 32;     // state columns per consumer wave
    constexpr int NCT = CPW / 16;           // 16-column tiles per consumer wave
    constexpr int NCONS = 4;                // consumer waves
    auto kslot = [](int64_t j) { return WY ? (int)(j & 1) : (int)(j % 3); };

    // the wave index is wave uniform: addresses built from it stay scalar
    const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;

    const int H = a.H;
    const int h = u.h;
    const ChainSpan sp = u.sp;
    const int64_t slot = u.slot;
    const int64_t n_chunks = (sp.t1 - sp.t0 + C - 1) / C;
    const int hk = h / (H / a.Hk);          // key head of this value head (grouped order)
    const int64_t rowK = (int64_t)a.Hk * K; // element stride between tokens of q, k
    const int64_t rowV = (int64_t)H * V;
    const uint32_t row_bytes_k = (uint32_t)(rowK * 2), row_bytes_v = (uint32_t)(rowV * 2);

    const bf16 *gq = static_cast<const bf16 *>(a.q);
    const bf16 *gk = static_cast<const bf16 *>(a.k);
    const bf16 *gv = static_cast<const bf16 *>(a.v);

    auto chunk_len = [&](int64_t j) -> int {
        const int64_t rem = sp.t1 - (sp.t0 + j * C);
        return rem < C ? (int)rem : C;
    };
    auto tok = [&](int64_t j, int r) -> int64_t { return sp.t0 + j * C + r; };

    if (wv < NCONS) {
        // =========================== consumers ===========================
        const bool is_M = !EMIT && cg == 0;
        const int col_w = (EMIT ? 64 * cg : 0) + CPW * wv;   // first state column
        f32x4 X[NCT][8];
        if (EMIT) {
            const float *hin = a.h_in;
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        X[n][t][e] = hin ? hin[(slot * K + 8 * lg + srow(t, e)) * V + col_w + 16 * n + li] : 0.f;
        } else {
            // M starts as the identity: state row 8g + srow(t, e) == column col_w + 16n + j
            const int diag = 8 * lg - col_w - li;
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        X[n][t][e] = (is_M && diag == 16 * n - srow(t, e)) ? 1.f : 0.f;
        }
        // value rows of this wave's columns, A layout of a 16x16x16 operand:
        // lane (i, g) holds v[16 c + i][col 4g .. 4g+3]
        uint2 vA[NCT][4];
        const uint32_t v_row = (uint32_t)li * row_bytes_v;
        auto load_v = [&](int64_t j) {
            if (is_M) {
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) vA[n][c] = make_uint2(0, 0);
                return;
            }
            if (WY) {
                // u rows of the chunk (every row present; zero past the chunk end)
                const __amdgpu_buffer_rsrc_t ur = rsrc(static_cast<const bf16 *>(a.wy_u) +
                                                       ((sp.chunk0 + j) * H + h) * (int64_t)C * V + col_w);
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        vA[n][c] = bload8(ur, (uint32_t)(16 * c + li) * (V * 2) + 2u * (16 * n + 4 * lg));
                return;
            }
            // rows past the chunk end read as zeros (the resource ends at row L)
            const int L = chunk_len(j);
            const __amdgpu_buffer_rsrc_t vr =
                rsrc_n(gv + tok(j, 0) * rowV + h * V + col_w, (uint32_t)L * row_bytes_v - 2u * (h * V + col_w));
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    vA[n][c] = bload8(vr, v_row + (uint32_t)(16 * c) * row_bytes_v + 2u * (16 * n + 4 * lg));
        };
        bf16x4 i16;   // identity, B operand of a 16x16x16 product
#pragma unroll
        for (int e = 0; e < 4; ++e) i16[e] = (bf16)((4 * lg + e == li) ? 1.f : 0.f);
        const uint32_t out_off = (uint32_t)((h * V + col_w + 4 * lg) * 2);   // bytes within a row

        if (n_chunks > 0) load_v(0);
        lds_barrier();   // iteration -2: k of chunk 0 loaded
        lds_barrier();   // iteration -1: chunk 0 prepared
        for (int64_t j = 0; j < n_chunks; ++j) {
            const int b2 = (int)(j & 1);
            const int L = chunk_len(j);
            // operand of Y = K X (recomputing) or of Y = w X (WY given)
            const bf16 *kR;
            if constexpr (WY) kR = sm.wR[b2];
            else kR = sm.kR[kslot(j)];
            // X as the operand reducing over the state rows
            bf16x8 hb[NCT][4];
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) hb[n][kk] = pack_pair(X[n][2 * kk], X[n][2 * kk + 1]);
            // -- Y = K X, k-block by k-block, the next block's fragments read
            // during the current block's products (each fragment feeds NCT
            // products, so one block ahead covers the LDS latency)
            f32x4 Y[NCT][4];
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int c = 0; c < 4; ++c) Y[n][c] = zero4();
            {
                bf16x8 ka[2][4];
#pragma unroll
                for (int c = 0; c < 4; ++c) ka[0][c] = ldv(kR, xoff(16 * c + li, lg));
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if (kk < 3)
#pragma unroll
                        for (int c = 0; c < 4; ++c) ka[(kk + 1) & 1][c] = ldv(kR, xoff(16 * c + li, 4 * (kk + 1) + lg));
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int n = 0; n < NCT; ++n) Y[n][c] = mma32(ka[kk & 1][c], hb[n][kk], Y[n][c]);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
                for (int i = 0; i < 12; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, NCT, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4 * NCT, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            // value tiles of this chunk in B layout, then the next chunk's loads;
            // T' and the decays read meanwhile
            const float *gam = sm.gam[b2];
            f32x4 Vt[NCT][4];
            bf16x8 ta[6];    // T' tiles (c, kk), kk <= c / 2
            f32x4 gv[4];     // gamma at rows 16c + 4g + e (B layout rows)
            float gr[4];     // gamma at row 16c + j (the rows of O^T's columns)
#pragma unroll
            for (int n = 0; n < NCT; ++n)
#pragma unroll
                for (int c = 0; c < 4; ++c) Vt[n][c] = mma16(__builtin_bit_cast(bf16x4, vA[n][c]), i16, zero4());
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                gv[c] = *reinterpret_cast<const f32x4 *>(&gam[16 * c + 4 * lg]);
                if (EMIT) gr[c] = gam[16 * c + li];
            }
#pragma unroll
            for (int i = 0; i < 6; ++i) {
                const int c = i < 1 ? 0 : i < 2 ? 1 : i < 4 ? 2 : 3, kk = (i == 3 || i == 5) ? 1 : 0;
                if constexpr (!WY) ta[i] = ldv(sm.tb[b2], noff(16 * c + li, 4 * kk + lg));
            }
            f32x4 D[NCT][4];
            if constexpr (WY) {
                // -- delta = u - w X (the row factors are inside u and w)
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) D[n][c] = Vt[n][c] - Y[n][c];
                if (j + 1 < n_chunks) load_v(j + 1);
            } else {
                // -- R = V - gamma (K X), packed as the operand reducing over the chunk
                bf16x8 R[NCT][2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int n = 0; n < NCT; ++n) {
                        f32x4 lo, hi;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            lo[e] = Vt[n][2 * kk][e] - gv[2 * kk][e] * Y[n][2 * kk][e];
                            hi[e] = Vt[n][2 * kk + 1][e] - gv[2 * kk + 1][e] * Y[n][2 * kk + 1][e];
                        }
                        R[n][kk] = pack_pair(lo, hi);
                    }
                if (j + 1 < n_chunks) load_v(j + 1);
                // -- D = T' R (delta = diag(beta) D)
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) D[n][c] = zero4();
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    const int c = i < 1 ? 0 : i < 2 ? 1 : i < 4 ? 2 : 3, kk = (i == 3 || i == 5) ? 1 : 0;
#pragma unroll
                    for (int n = 0; n < NCT; ++n) D[n][c] = mma32(ta[i], R[n][kk], D[n][c]);
                }
            }
            // D as the operand reducing over the chunk, for both products that
            // follow: the kT tile carries the row factors of the state update and
            // the attn tile those of the output
            bf16x8 dk[NCT][2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int n = 0; n < NCT; ++n) dk[n][kk] = pack_pair(D[n][2 * kk], D[n][2 * kk + 1]);
            // -- X = gamma_C X + K^T diag(exp(G_C - G)) delta = gamma_C X + (K^T diag(kdec)) D,
            // the k^T fragments of two row tiles read ahead of their products
            const float gc = gam[63];
            {
                bf16x8 kt[2][4];   // [t & 1][2 (t / 2 parity) + kk] fragments of row tiles
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) kt[0][2 * t + kk] = ldv(sm.kT[b2], noff(16 * t + li, 4 * kk + lg));
#pragma unroll
                for (int tp = 0; tp < 4; ++tp) {   // row tiles 2tp, 2tp + 1
                    if (tp < 3)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int kk = 0; kk < 2; ++kk)
                                kt[(tp + 1) & 1][2 * t + kk] =
                                    ldv(sm.kT[b2], noff(16 * (2 * tp + 2 + t) + li, 4 * kk + lg));
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int n = 0; n < NCT; ++n) {
                            X[n][2 * tp + t] *= gc;
#pragma unroll
                            for (int kk = 0; kk < 2; ++kk)
                                X[n][2 * tp + t] = mma32(kt[tp & 1][2 * t + kk], dk[n][kk], X[n][2 * tp + t]);
                        }
                }
            }
            if (EMIT) {
                // -- O^T = X^T Q^T + D^T (attn diag(beta))^T, formed transposed: the
                // operands are the registers of X (B layout of X = A layout of X^T)
                // and the q row fragments (A layout of Q = B layout of Q^T), and
                // tile c of O^T leaves lane (j, g) holding row 16c + j, columns
                // 4g .. 4g+3 of O -- eight contiguous bytes of an output row.
                // (attn diag(beta) when recomputing: the attn tile carries beta on
                // its columns; attn alone when the WY factors are given.)
                f32x4 O[NCT][4];
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) O[n][c] = zero4();
                bf16x8 qa[2][4];
#pragma unroll
                for (int c = 0; c < 4; ++c) qa[0][c] = ldv(sm.qR[b2], xoff(16 * c + li, lg));
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if (kk < 3)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            qa[(kk + 1) & 1][c] = ldv(sm.qR[b2], xoff(16 * c + li, 4 * (kk + 1) + lg));
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int n = 0; n < NCT; ++n) O[n][c] = mma32(hb[n][kk], qa[kk & 1][c], O[n][c]);
                }
                bf16x8 at6[6];
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    const int c = i < 1 ? 0 : i < 2 ? 1 : i < 4 ? 2 : 3, kk = (i == 3 || i == 5) ? 1 : 0;
                    at6[i] = ldv(sm.attn[b2], noff(16 * c + li, 4 * kk + lg));
                }
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) O[n][c] *= gr[c];
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    const int c = i < 1 ? 0 : i < 2 ? 1 : i < 4 ? 2 : 3, kk = (i == 3 || i == 5) ? 1 : 0;
#pragma unroll
                    for (int n = 0; n < NCT; ++n) O[n][c] = mma32(dk[n][kk], at6[i], O[n][c]);
                }
                // rows past the chunk end fall outside the resource: dropped
                const __amdgpu_buffer_rsrc_t orr =
                    rsrc_n(static_cast<bf16 *>(a.o) + tok(j, 0) * rowV, (uint32_t)L * (uint32_t)(rowV * 2));
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint2 v = __builtin_bit_cast(uint2, to4(O[n][c]));
                        bstore8(orr, (uint32_t)(16 * c + li) * (uint32_t)(rowV * 2) + out_off + 32u * n, v);
                    }
            }
            lds_barrier();
        }
        // chain end: final state (emit, last segment) or the pair (M_r, U_r) (carry)
        if (EMIT) {
            if (a.h_out && u.final_state) {
                // (batch mode: the chain's sequence, computed here rather than
                // kept live through the loop)
                const int64_t so = PACKED ? u.out_slot : (int64_t)sp.seq * H + h;
#pragma unroll
                for (int n = 0; n < NCT; ++n)
#pragma unroll
                    for (int t = 0; t < 8; ++t)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            a.h_out[(so * K + 8 * lg + srow(t, e)) * V + col_w + 16 * n + li] = X[n][t][e];
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
                        dst[(slot * K + 8 * lg + srow(t, e)) * ld + col_w + 16 * n + li] = X[n][t][e];
        }
        return;
    }

    // ============================ producers ============================
    // Iteration it = -2 .. n-1 (one barrier each, matching the consumers' two
    // prologue barriers and one per chunk): the loader stores chunk it+2 (and
    // has the loads of chunk it+3, emitting also it+4, in flight); waves 4, 6,
    // 7 prepare chunk it+1.  The two waves that keep loads in flight across a
    // barrier (loader, q) run their loop unrolled by two so each register set
    // has a fixed home, and always issue a load (of the last chunk when past
    // the end).
    const int role = wv - 4;
    if (n_chunks == 0 || role < 0) {
        for (int64_t it = -2; it < n_chunks; ++it) lds_barrier();
        return;
    }
    auto clampj = [&](int64_t j) { return j < n_chunks ? j : n_chunks - 1; };
    if (role == 1) {
        // ---------------- loader: k rows, g, beta; two register sets ----------------
        uint4 kA_[16], kB_[16];
        float gA, bA, gB, bB;
        auto issue = [&](uint4 (&t)[16], float &gv_, float &bv_, int64_t j) {
            const int L = chunk_len(j);
            load_rows(t, gk + tok(j, 0) * rowK + hk * K, row_bytes_k, L, lane);
            const int64_t t0 = tok(j, 0) * H + h;
            const uint32_t go = min((uint32_t)lane, (uint32_t)(L - 1)) * (uint32_t)(4 * H);
            gv_ = bload4f(rsrc(a.g + t0), go);
            bv_ = bload4f(rsrc(a.beta + t0), go);
        };
        if constexpr (EMIT) {
            // Emitting: chunk j's rows are stored at iteration j-2, and the same
            // registers then take the loads of chunk j+2, so each load has about
            // two iterations to arrive (the carrying workgroups, whose producers
            // have less to do, keep one, below).
            //
            // The rest of chunk j's preparation once its rows are in LDS; gl, bl
            // are g and beta of its rows (0 past the chunk end).  The lane index
            // is made opaque here, so the LDS addresses are formed at each chunk
            // instead of being held in registers across the loop while two
            // chunks' loads are in flight.
            auto prep = [&](float gl, float bl, int64_t j) {
                const int b3 = kslot(j), b2 = (int)(j & 1);
                int ln = lane;
                asm volatile("" : "+v"(ln));
                const int li = ln & 15, lg = ln >> 4;
                const float g2 = wave_cumsum(gl) * kLog2e;
                sm.G2[b2][ln] = g2;
                if constexpr (!WY) {
                    sm.B[b2][ln] = bl;
                    // log2(0) = -inf: padded columns of attn vanish
                    sm.Gb[b2][ln] = g2 - __builtin_amdgcn_logf(fabsf(bl));
                    const bool neg = __builtin_amdgcn_ballot_w64(bl < 0.f) != 0;
                    if (ln == 0) sm.negb[b2] = neg;
                    // the k rows back in MFMA operand layout (this wave's own
                    // writes), read as the Gram consumes them
                    const bf16 *kR = sm.kR[b3];
                    gram_to_ab([&](int c, int kk) { return ldv(kR, xoff(16 * c + li, 4 * kk + lg)); }, sm.G2[b2],
                               sm.B[b2], sm.ab[b2], ln);
                }
            };
            auto step = [&](uint4 (&t)[16], float &gv_, float &bv_, int64_t j) {
                const bool live = j < n_chunks;
                float gl = 0.f, bl = 0.f;
                if (live) {
                    store_rows(sm.kR[kslot(j)], t, lane);
                    const bool in = lane < chunk_len(j);
                    gl = in ? gv_ : 0.f;
                    bl = in ? bv_ : 0.f;
                }
                issue(t, gv_, bv_, clampj(j + 2));
                if (live) prep(gl, bl, j);
            };
            issue(kA_, gA, bA, 0);
            __builtin_amdgcn_sched_barrier(0);   // chunk 0's loads first: the wait counts rely on it
            issue(kB_, gB, bB, clampj(1));
            // iterations in pairs, then the odd one: no exit between the two
            // halves, so on every path the other set's loads are the later ones
            // and each half waits for its own set only
            int64_t it = -2;
            for (; it + 1 < n_chunks; it += 2) {
                step(kA_, gA, bA, it + 2);
                lds_barrier();
                step(kB_, gB, bB, it + 3);
                lds_barrier();
            }
            if (it < n_chunks) {
                step(kA_, gA, bA, it + 2);
                lds_barrier();
            }
        } else {
            // Carrying: the loads of chunk j+3 go out at iteration j and are
            // stored at the next.
            auto store = [&](const uint4 (&t)[16], float gv_, float bv_, int64_t j) {
                const int b3 = kslot(j), b2 = (int)(j & 1);
                const int L = chunk_len(j);
                store_rows(sm.kR[b3], t, lane);
                // rows past the chunk end get g = 0, beta = 0
                const float g2 = wave_cumsum(lane < L ? gv_ : 0.f) * kLog2e;
                sm.G2[b2][lane] = g2;
                if constexpr (!WY) {
                    // the k rows back in MFMA operand layout (this wave's own writes)
                    bf16x8 kt[4][4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) kt[c][kk] = ldv(sm.kR[b3], xoff(16 * c + li, 4 * kk + lg));
                    const float bl = lane < L ? bv_ : 0.f;
                    sm.B[b2][lane] = bl;
                    sm.Gb[b2][lane] = g2 - __builtin_amdgcn_logf(fabsf(bl));
                    const bool neg = __builtin_amdgcn_ballot_w64(bl < 0.f) != 0;
                    if (lane == 0) sm.negb[b2] = neg;
                    gram_to_ab([&](int c, int kk) { return kt[c][kk]; }, sm.G2[b2], sm.B[b2], sm.ab[b2], lane);
                }
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
        }
        return;
    }
    if (role == 2) {
        // -------- q rows (one chunk ahead) -> qR, and attn from the Gram k q^T --------
        if (!EMIT) {
            for (int64_t it = -2; it < n_chunks; ++it) lds_barrier();
            return;
        }
        uint4 qA_[16], qB_[16];
        auto issue = [&](uint4 (&t)[16], int64_t j) {
            load_rows(t, gq + tok(j, 0) * rowK + hk * K, row_bytes_k, chunk_len(j), lane);
        };
        auto work = [&](const uint4 (&qraw)[16], int64_t jn) {
            const int b2 = (int)(jn & 1), b3 = kslot(jn);
            const int L = chunk_len(jn);
            const bf16 *kR = sm.kR[b3];
            store_rows(sm.qR[b2], qraw, lane);

            const float *G2 = sm.G2[b2];
            (void)L;
            // Gram block (b, a) of K Q^T: lane (j, g) element e holds
            // k_{16b+4g+e} . q_{16a+j} = raw attn[r = 16a + j][s = 16b + 4g + e]
            f32x4 acc[10];
#pragma unroll
            for (int i = 0; i < 10; ++i) acc[i] = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 qa[4], kb[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    qa[c] = ldv(sm.qR[b2], xoff(16 * c + li, 4 * kk + lg));
                    kb[c] = ldv(kR, xoff(16 * c + li, 4 * kk + lg));
                }
                int i = 0;
#pragma unroll
                for (int aa = 0; aa < 4; ++aa)
#pragma unroll
                    for (int bb = 0; bb <= aa; ++bb, ++i) acc[i] = mma32(kb[bb], qa[aa], acc[i]);
            }
            // attn diag(beta) when recomputing (the factor that multiplies D), from
            // the column exponents G2 - log2|beta| (beta = 0 zeroes padded
            // columns), with beta multiplied in instead when some beta of the
            // chunk is negative; plain attn for the WY factors (beta is inside
            // u and w)
            bf16x4 at[4][4];
            auto form = [&](const float *Gcol, bool times_beta) {
                int i = 0;
#pragma unroll
                for (int aa = 0; aa < 4; ++aa) {
                    const int r = 16 * aa + li;
                    const float Gr = G2[r];
#pragma unroll
                    for (int bb = 0; bb <= aa; ++bb, ++i) {
                        const f32x4 Gs = *reinterpret_cast<const f32x4 *>(&Gcol[16 * bb + 4 * lg]);
                        f32x4 sc = acc[i];
                        if constexpr (!WY)
                            if (times_beta) sc *= *reinterpret_cast<const f32x4 *>(&sm.B[b2][16 * bb + 4 * lg]);
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            // causal mask on the diagonal blocks only
                            const int s_ = 16 * bb + 4 * lg + e;
                            v[e] = (bb < aa || s_ <= r) ? ex2(Gr - Gs[e]) * sc[e] : 0.f;
                        }
                        at[aa][bb] = to4(v);
                    }
                }
            };
            if constexpr (WY) {
                form(G2, false);
            } else {
                if (__builtin_amdgcn_readfirstlane(sm.negb[b2])) form(G2, true);
                else form(sm.Gb[b2], false);
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
    if (WY && role == 0) {
        // -------- w rows of the WY workspace (one chunk ahead) -> wR --------
        uint4 wA_[16], wB_[16];
        auto issue = [&](uint4 (&t)[16], int64_t j) {
            load_rows(t, static_cast<const bf16 *>(a.wy_w) + ((sp.chunk0 + j) * H + h) * (int64_t)C * K, K * 2, C,
                      lane);
        };
        auto put = [&](const uint4 (&t)[16], int64_t jn) {
            if constexpr (WY) store_rows(sm.wR[jn & 1], t, lane);
        };
        issue(wA_, 0);
        lds_barrier();   // iteration -2
        for (int64_t it = -1; it < n_chunks; it += 2) {
            issue(wB_, clampj(it + 2));
            if (it + 1 < n_chunks) put(wA_, it + 1);
            lds_barrier();
            if (it + 1 >= n_chunks) break;
            issue(wA_, clampj(it + 3));
            if (it + 2 < n_chunks) put(wB_, it + 2);
            lds_barrier();
        }
        return;
    }
    const InvMasks im = inv_masks(lane);   // (wave 4's inverse)
    // identity selectors (B operands) picking columns 0-15 / 16-31 of a 32-wide block
    bf16x8 id0, id1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool hit = 4 * lg + (e & 3) == li;
        id0[e] = (bf16)((hit && (e >> 2) == 0) ? 1.f : 0.f);
        id1[e] = (bf16)((hit && (e >> 2) == 1) ? 1.f : 0.f);
    }
    for (int64_t it = -2; it < n_chunks; ++it) {
        const int64_t jn = it + 1;   // chunk being prepared
        if (jn >= 0 && jn < n_chunks) {
            const int b2 = (int)(jn & 1), b3 = kslot(jn);
            const bf16 *kR = sm.kR[b3];
            const float *G2 = sm.G2[b2];
            if (role == 3) {
                // ---- per-row factors, and K^T diag(kdec) by identity products
                const float g2 = G2[lane];
                sm.gam[b2][lane] = ex2(g2);
                if constexpr (WY) {
                    sm.kdec[b2][lane] = ex2(G2[63] - g2);
                } else {
                    sm.kdec[b2][lane] = ex2(G2[63] - g2) * sm.B[b2][lane];
                }
                // kdec at rows 16c + 4g + e (this wave's own writes, read back)
                f32x4 kd[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) kd[c] = *reinterpret_cast<const f32x4 *>(&sm.kdec[b2][16 * c + 4 * lg]);
                bf16 *kT = sm.kT[b2];
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const bf16x8 id = (n & 1) ? id1 : id0;
                    f32x4 d[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        d[c] = mma32(ldv(kR, xoff(16 * c + li, 4 * (n >> 1) + lg)), id, zero4());
                    }
                    // lane (j, g) of d[c] holds k[16c + 4g + e][16n + j]
#pragma unroll
                    for (int c = 0; c < 4; ++c)
#pragma unroll
                        for (int e = 0; e < 4; ++e) d[c][e] *= kd[c][e];
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
                        stv(kT, noff(16 * n + li, 4 * kk + lg), pack_pair(d[2 * kk], d[2 * kk + 1]));
                }
            } else {
                // ---- role 0: T' = (I + A0 diag(beta))^{-1} from the loader's Gram tiles
                if constexpr (!WY) invert_tprime(sm.ab[b2], G2, sm.B[b2], sm.tb[b2], nullptr, lane, im);
            }
        }
        lds_barrier();
    }
}

// PACKED: the chains are work items of a packed problem (a separate
// instantiation keeps the batch kernels' code as it is).
template <bool EMIT, bool WY, bool PACKED>
__global__ __launch_bounds__(NT, 1) void scan_mfma_kernel(ScanArgs a, int n_units) {
    __shared__ Lds<WY> sm;
    const int unit = unit_of_block(blockIdx.x);
    if (unit >= n_units) return;
    const int h = unit % a.H, chain = unit / a.H;
    const UnitRef r = PACKED ? packed_unit(a.ct, chain, h, a.H, C) : batch_unit(a.ct, chain, h, a.H, C, !EMIT);
    if (r.carry == EMIT) return;   // an item of the other kind (the host never lists one)
    scan_body<EMIT, WY, PACKED>(sm, a, scan_unit(r, h), half_of_block(blockIdx.x));
}

// One launch for segment 0 of every sequence emitted (from h_in, outputs o,
// final state h_out) beside segments 1 .. R-1 carried (pairs in slots 0 .. R-2
// of M_out, U_out).  Batch mode: a holds the chain table of all R segments and
// the carrying pass's outputs; the first emit_blocks workgroups emit.  Packed
// mode: every pointer is in a, and each work item says whether it emits or
// carries (emit_blocks is unused).
template <bool WY, bool PACKED>
__global__ __launch_bounds__(NT, 1) void scan_mfma_head_kernel(ScanArgs a, const float *h_in, void *o, float *h_out,
                                                               int emit_blocks) {
    __shared__ Lds<WY> sm;
    const int R = a.ct.n_seg, N = a.ct.n_seqs, H = a.H;
    if (PACKED) {
        const int unit = unit_of_block(blockIdx.x);
        if (unit >= a.ct.n_items * H) return;
        const int h = unit % H;
        const UnitRef r = packed_unit(a.ct, unit / H, h, H, C);
        if (r.carry) scan_body<false, WY, true>(sm, a, scan_unit(r, h), half_of_block(blockIdx.x));
        else scan_body<true, WY, true>(sm, a, scan_unit(r, h), half_of_block(blockIdx.x));
        return;
    }
    const bool emitting = (int)blockIdx.x < emit_blocks;
    const int bid = emitting ? (int)blockIdx.x : (int)blockIdx.x - emit_blocks;
    const int unit = unit_of_block(bid);
    ScanUnit u;
    u.h = unit % H;
    if (emitting) {
        if (unit >= N * H) return;
        const int seq = unit / H;
        u.sp = chain_span(a.ct, seq * R, C);
        u.slot = (int64_t)seq * H + u.h;
        u.final_state = true;
        ScanArgs e = a;
        e.h_in = h_in;
        e.o = o;
        e.h_out = h_out;
        e.M_out = e.U_out = nullptr;
        scan_body<true, WY, false>(sm, e, u, half_of_block(bid));
    } else {
        if (unit >= N * (R - 1) * H) return;
        const int c = unit / H, seq = c / (R - 1), seg = 1 + c % (R - 1);
        u.sp = chain_span(a.ct, seq * R + seg, C);
        u.slot = ((int64_t)(seg - 1) * N + seq) * H + u.h;
        u.final_state = false;
        scan_body<false, WY, false>(sm, a, u, half_of_block(bid));
    }
}

}  // namespace

bool mfma_scan_available(int K_, int V_, int C_, int dtype) {
    return K_ == K && V_ == V && C_ == C && dtype == GDN_BF16;
}

hipError_t launch_scan_mfma(int K_, int V_, int C_, int dtype, bool carry, const ScanArgs &a,
                            hipStream_t s, bool *handled) {
    *handled = false;
    if (!mfma_scan_available(K_, V_, C_, dtype)) return hipSuccess;
    *handled = true;
    const int64_t units = (int64_t)a.n_chains * a.H;
    if (units == 0) return hipSuccess;
    const int64_t grid = ((units + 7) / 8) * 16;   // two column halves, 8 ids apart
    const dim3 g((unsigned)grid), b(NT);
    const bool wy = a.wy_w != nullptr;
    if (a.ct.packed) {
        if (carry && wy) hipLaunchKernelGGL((scan_mfma_kernel<false, true, true>), g, b, 0, s, a, (int)units);
        else if (carry) hipLaunchKernelGGL((scan_mfma_kernel<false, false, true>), g, b, 0, s, a, (int)units);
        else if (wy) hipLaunchKernelGGL((scan_mfma_kernel<true, true, true>), g, b, 0, s, a, (int)units);
        else hipLaunchKernelGGL((scan_mfma_kernel<true, false, true>), g, b, 0, s, a, (int)units);
        return hipGetLastError();
    }
    if (carry && wy) hipLaunchKernelGGL((scan_mfma_kernel<false, true, false>), g, b, 0, s, a, (int)units);
    else if (carry) hipLaunchKernelGGL((scan_mfma_kernel<false, false, false>), g, b, 0, s, a, (int)units);
    else if (wy) hipLaunchKernelGGL((scan_mfma_kernel<true, true, false>), g, b, 0, s, a, (int)units);
    else hipLaunchKernelGGL((scan_mfma_kernel<true, false, false>), g, b, 0, s, a, (int)units);
    return hipGetLastError();
}

hipError_t launch_scan_head_mfma(int K_, int V_, int C_, int dtype, const ScanArgs &a, const float *h_in, void *o,
                                 float *h_out, hipStream_t s, bool *handled) {
    *handled = false;
    if (!mfma_scan_available(K_, V_, C_, dtype)) return hipSuccess;
    *handled = true;
    int64_t emit_blocks, carry_blocks;
    if (a.ct.packed) {
        // every pointer is in a; the items carry their kinds
        const int64_t units = (int64_t)a.ct.n_items * a.H;
        if (units == 0) return hipSuccess;
        emit_blocks = ((units + 7) / 8) * 16;
        carry_blocks = 0;
    } else {
        const int64_t N = a.ct.n_seqs, R = a.ct.n_seg;
        const int64_t emit_units = N * a.H, carry_units = N * (R - 1) * a.H;
        if (emit_units == 0) return hipSuccess;
        emit_blocks = ((emit_units + 7) / 8) * 16;
        carry_blocks = ((carry_units + 7) / 8) * 16;
    }
    const dim3 g((unsigned)(emit_blocks + carry_blocks)), b(NT);
    const bool pk = a.ct.packed != 0;
    if (a.wy_w && pk) hipLaunchKernelGGL((scan_mfma_head_kernel<true, true>), g, b, 0, s, a, h_in, o, h_out, 0);
    else if (pk) hipLaunchKernelGGL((scan_mfma_head_kernel<false, true>), g, b, 0, s, a, h_in, o, h_out, 0);
    else if (a.wy_w)
        hipLaunchKernelGGL((scan_mfma_head_kernel<true, false>), g, b, 0, s, a, h_in, o, h_out, (int)emit_blocks);
    else hipLaunchKernelGGL((scan_mfma_head_kernel<false, false>), g, b, 0, s, a, h_in, o, h_out, (int)emit_blocks);
    return hipGetLastError();
}

}  // namespace gdn
