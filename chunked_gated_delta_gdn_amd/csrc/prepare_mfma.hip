// Matrix-core per-chunk WY preparation for bf16 inputs at K = V = 128, C = 64
// (the w and u of the affine chunk map in the MaxText PR "Add context
// parallelism to the Gated Delta Net", section "Why"; the chunk_prepare step of
// section "Implementation"):
//   w = T diag(beta gamma) K,   u = T diag(beta) V,   T = (I + A)^{-1},
//   A[r,s] = beta_r exp(G_r - G_s) k_r.k_s (s < r),   gamma_s = exp(G_s).
// With A = diag(beta) A0 and T diag(beta) = diag(beta) T', where
// T' = (I + A0 diag(beta))^{-1} (the identity used by the scan), this is
//   w = diag(beta) (T' diag(gamma)) K,   u = diag(beta) T' V.
//
// One workgroup of 4 waves per (chunk, head); chunks are independent, so the
// grid is n_chunks * H workgroups and several share a CU.
//   * all waves load their quarter of the k and v rows (whole 256-byte rows)
//     into operand-layout LDS tiles; wave 0 also the decays and beta;
//   * the four waves split the ten Gram tiles, then invert one diagonal 16 x 16
//     block of T' each; wave 0 forms the off-diagonal blocks and writes T'
//     and T' diag(gamma) (all on MFMA);
//   * every wave then computes 2 + 2 row blocks of w^T = K^T (T' diag(gamma))^T
//     and u^T = V^T T'^T.  The K^T / V^T operands come from the row tiles by
//     transposing LDS reads; an accumulator of w^T holds, per lane, 4
//     consecutive keys of one chunk row, so rows are scaled by beta and staged
//     as 8-byte runs in the (by then free) row tiles, from where the w and u
//     blocks go out as whole rows, 16 bytes per lane (scattered 8-byte stores
//     cost the stream about 15%).
// Rows past the end of a ragged chunk have beta = 0 and come out as zeros.
#include "dev_common.h"
#include "gdn_internal.h"
#include "mfma_tile.h"

namespace gdn {
namespace {
using namespace mfma;

constexpr int K = 128, V = 128, C = 64;
constexpr int NTP = 256;   // 4 waves

struct PrepLds {
    bf16 kR[C * K];        // k rows, wide tiles
    bf16 vR[C * V];        // v rows, wide tiles
    union {
        bf16 tb[C * C];    // T'
        struct {           // before T' is written: the diagonal inverses, per lane
            uint2 P[4][64];
            f32x4 Qf[4][64];
        } dg;
    };
    union {
        uint2 ab[10][64];  // Gram tiles (see gram_to_ab), read by invert_tprime first,
        bf16 tg[C * C];    // then overwritten by T' diag(gamma): 3 workgroups fit a CU
    };
    float G2[C];           // cumulative log2-decay (zero past the chunk end)
    float B[C];            // beta (zero past the chunk end)
};

// Quarter (rows 16 w .. 16 w + 15) of a 64-row tile: load m = 4w .. 4w+3 of
// load_rows, the same lane mapping and row clamping.
__device__ __forceinline__ void load_quarter(uint4 (&t)[4], const bf16 *base, uint32_t row_bytes, int L,
                                             int lane, int w) {
    const __amdgpu_buffer_rsrc_t r = rsrc(base);
    const uint32_t lim = (uint32_t)(L - 1) * row_bytes;
    const uint32_t own = (uint32_t)(lane >> 4) * row_bytes;
    const uint32_t col = 16u * (lane & 15);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        t[m] = bload16(r, min(own + (uint32_t)(4 * (4 * w + m)) * row_bytes, lim) + col, 0);
}
__device__ __forceinline__ void store_quarter(bf16 *tile, const uint4 (&t)[4], int lane, int w) {
    const int s = lane & 15;
    const int q0 = 4 * (s >> 2) + 2 * (s & 1), within = 8 * ((s >> 1) & 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int r = 4 * (4 * w + m) + (lane >> 4);
        char *b = reinterpret_cast<char *>(tile);
        *reinterpret_cast<uint2 *>(b + woff(r, q0) + within) = make_uint2(t[m].x, t[m].y);
        *reinterpret_cast<uint2 *>(b + woff(r, q0 + 1) + within) = make_uint2(t[m].z, t[m].w);
    }
}

__global__ __launch_bounds__(NTP) void prepare_mfma_kernel(PrepArgs a) {
    __shared__ PrepLds sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int H = a.H;
    const int h = blockIdx.x % H;
    const int64_t chunk = blockIdx.x / H;

    // the chunk's sequence and first token
    int64_t tc, tend;
    if (a.ct.packed) {
        int lo = 0, hi = a.ct.n_seqs - 1;   // last n with chunk_start[n] <= chunk
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.ct.chunk_start[mid] <= chunk) lo = mid;
            else hi = mid - 1;
        }
        tc = a.ct.seq_start[lo] + (chunk - a.ct.chunk_start[lo]) * C;
        tend = a.ct.seq_start[lo + 1];
    } else {
        const int64_t per = (a.ct.seq_len + C - 1) / C;
        const int64_t n = chunk / per;
        tc = n * a.ct.seq_len + (chunk % per) * C;
        tend = (n + 1) * a.ct.seq_len;
    }
    const int L = (int)((tend - tc) < C ? (tend - tc) : C);
    const int64_t rowK = (int64_t)a.Hk * K, rowV = (int64_t)H * V;
    const int hk = h / (H / a.Hk);   // key head of this value head (grouped order)

    {
        uint4 tk[4], tv[4];
        load_quarter(tk, static_cast<const bf16 *>(a.k) + tc * rowK + hk * K, (uint32_t)(rowK * 2), L, lane, wv);
        load_quarter(tv, static_cast<const bf16 *>(a.v) + tc * rowV + h * V, (uint32_t)(rowV * 2), L, lane, wv);
        if (wv == 0) {
            const uint32_t go = min((uint32_t)lane, (uint32_t)(L - 1)) * (uint32_t)(4 * H);
            const float gl = bload4f(rsrc(a.g + tc * H + h), go);
            const float bl = bload4f(rsrc(a.beta + tc * H + h), go);
            sm.G2[lane] = wave_cumsum(lane < L ? gl : 0.f) * kLog2e;
            sm.B[lane] = lane < L ? bl : 0.f;
        }
        store_quarter(sm.kR, tk, lane, wv);
        store_quarter(sm.vR, tv, lane, wv);
    }
    __syncthreads();
    // the Gram tiles, split over the waves (blocks numbered as in gram_to_ab)
    {
        auto kt = [&](int c, int kk) { return ldv(sm.kR, woff(16 * c + li, 4 * kk + lg)); };
        switch (wv) {
            case 0: gram_to_ab<0x111>(kt, sm.G2, sm.B, sm.ab, lane); break;
            case 1: gram_to_ab<0x222>(kt, sm.G2, sm.B, sm.ab, lane); break;
            case 2: gram_to_ab<0x044>(kt, sm.G2, sm.B, sm.ab, lane); break;
            default: gram_to_ab<0x088>(kt, sm.G2, sm.B, sm.ab, lane); break;
        }
    }
    __syncthreads();
    // diagonal block wv of T'
    {
        auto one = [&](const int (&b)[1]) {
            bf16x4 P[1];
            f32x4 Qf[1];
            diag_inverse(b, sm.ab, sm.G2, sm.B, lane, inv_masks(lane), P, Qf);
            sm.dg.P[b[0]][lane] = __builtin_bit_cast(uint2, P[0]);
            sm.dg.Qf[b[0]][lane] = Qf[0];
        };
        switch (wv) {
            case 0: { const int b[1] = {0}; one(b); break; }
            case 1: { const int b[1] = {1}; one(b); break; }
            case 2: { const int b[1] = {2}; one(b); break; }
            default: { const int b[1] = {3}; one(b); break; }
        }
    }
    __syncthreads();
    if (wv == 0) {
        bf16x4 P[4];
        f32x4 Qf[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            P[a] = __builtin_bit_cast(bf16x4, sm.dg.P[a][lane]);
            Qf[a] = sm.dg.Qf[a][lane];
        }
        // the diagonal inverses share memory with tb: offdiag_store reads
        // everything before its first write
        offdiag_store(sm.ab, sm.G2, P, Qf, sm.tb, sm.tg, lane);
    }
    __syncthreads();

    // w^T (from K, T' diag(gamma)) and u^T (from V, T'): this wave's row blocks
    // t = 2 wv, 2 wv + 1 of each.  A operand: k-slots 0-3 of lane (i, g) of
    // block (t, kk) are src[32kk + 4g + e][16t + i], slots 4-7 the same 16 rows
    // further, so lane s addresses the 4 elements 16t + 4(s & 3) .. +3 of row
    // 32kk + 4(s >> 4) + (s & 15) / 4 (and 16 rows on).
    const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2), tr_q = lane & 3;
    float bc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bc[c] = sm.B[16 * c + li];
    const size_t blk = (size_t)chunk * H + h;
    bf16x4 outv[2][2][4];   // [w or u][tt][c]: out[16c + li][16(2 wv + tt) + 4 lg .. +3]
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const bf16 *src = which == 0 ? sm.kR : sm.vR;
        const bf16 *rt = which == 0 ? sm.tg : sm.tb;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * wv + tt;
            const int q = 4 * (t >> 1) + tr_q, wb = 8 * (t & 1);
            bf16x8 at[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                at[kk] = join(ldtr(src, woff(32 * kk + tr_row, q) + wb), ldtr(src, woff(32 * kk + 16 + tr_row, q) + wb));
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f32x4 acc = zero4();
                // T' is lower triangular: rows 0-31 have no columns 32-63 (and the
                // tiles leave that block unwritten)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    if (kk <= (c >> 1)) acc = mma32(at[kk], ldv(rt, noff(16 * c + li, 4 * kk + lg)), acc);
                f32x4 sv;
#pragma unroll
                for (int e = 0; e < 4; ++e) sv[e] = acc[e] * bc[c];
                outv[which][tt][c] = to4(sv);
            }
        }
    }
    // stage the rows in the row tiles (every read of them is done): row r, 16-byte
    // chunk q at chunk q ^ (r & 15) of a 256-byte row
    __syncthreads();
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        char *stg = reinterpret_cast<char *>(which == 0 ? sm.kR : sm.vR);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int r = 16 * c + li, q = 2 * (2 * wv + tt) + (lg >> 1);
                *reinterpret_cast<uint2 *>(stg + r * 256 + ((q ^ (r & 15)) << 4) + 8 * (lg & 1)) =
                    __builtin_bit_cast(uint2, outv[which][tt][c]);
            }
    }
    __syncthreads();
    // whole rows out: the w and u blocks of this (chunk, head) are contiguous
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const char *stg = reinterpret_cast<const char *>(which == 0 ? sm.kR : sm.vR);
        char *dst = reinterpret_cast<char *>(static_cast<bf16 *>(which == 0 ? a.wy_w : a.wy_u) +
                                             blk * C * (which == 0 ? K : V));
        // (streaming stores: the workspace is written once here and read once by
        // the scan, and exceeds the last-level cache at long sequences)
        typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e16 = m * NTP + tid, r = e16 >> 4, q = e16 & 15;
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4v *>(stg + r * 256 + ((q ^ (r & 15)) << 4)),
                                        reinterpret_cast<u32x4v *>(dst + 16 * e16));
        }
    }
}

}  // namespace

bool mfma_prepare_available(int K_, int V_, int C_, int dtype) {
    return K_ == K && V_ == V && C_ == C && dtype == GDN_BF16;
}

hipError_t launch_prepare_mfma(const PrepArgs &a, hipStream_t s) {
    const int64_t n = a.n_chunks * a.H;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(prepare_mfma_kernel, dim3((unsigned)n), dim3(NTP), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
