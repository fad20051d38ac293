// mfma_tile.h -- register, LDS and load helpers shared by the matrix-core
// kernels (the chunked scan and the per-chunk WY preparation) at
// K = V = 128, C = 64, bf16 operands with fp32 accumulation on gfx950, and the
// two per-chunk building blocks both use: the decayed Gram tiles of A and the
// inverse T' = (I + A0 diag(beta))^{-1} (see scan_mfma.hip for the algebra).
#ifndef GDN_MFMA_TILE_H
#define GDN_MFMA_TILE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
namespace mfma {

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

// Round to bf16 (nearest even) two values at a time into one 32-bit register
// (a single v_cvt_pk_bf16_f32), then reinterpret: converting whole bf16
// vectors that feed an MFMA otherwise costs a conversion and a permute per
// element.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ bf16x4 to4(const f32x4 &x) {
    return __builtin_bit_cast(bf16x4, make_uint2(cvt2(x[0], x[1]), cvt2(x[2], x[3])));
}
__device__ __forceinline__ bf16x8 join(const bf16x4 &lo, const bf16x4 &hi) {
    const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(bf16x8, make_uint4(l.x, l.y, h.x, h.y));
}
// Two accumulator tiles (rows 0-15, 16-31 of a 32-row block) -> the bf16
// operand that reduces over those 32 rows.
__device__ __forceinline__ bf16x8 pack_pair(const f32x4 &lo, const f32x4 &hi) {
    return __builtin_bit_cast(bf16x8, make_uint4(cvt2(lo[0], lo[1]), cvt2(lo[2], lo[3]),
                                                 cvt2(hi[0], hi[1]), cvt2(hi[2], hi[3])));
}
__device__ __forceinline__ bf16x8 as8(const uint4 &u) { return __builtin_bit_cast(bf16x8, u); }

// Decays are kept as log2 values, so exp(G_r - G_s) is one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that waits for this wave's LDS operations only (global
// loads issued earlier stay in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS tiles.  A row of a "wide" tile holds 128 bf16 (16 chunks of 16 B), a row
// of a "narrow" tile 64 bf16 (8 chunks).  Within a 32-element block, chunk g
// holds the k-slots 8g .. 8g+7 that lane group g feeds to a 16x16x32 MFMA.
// Wide tiles written by store_rows hold them in natural order (k-slot 8g + e
// is element 8g + e of the block); the other tiles, whose reduction runs over
// the tokens of a chunk, hold logical elements 4g .. 4g+3 and 16+4g .. 16+4g+3
// there, so that two accumulator tiles (rows 0-15 and 16-31) are directly the
// operand reducing over those 32 rows (pack_pair).
// The 16-byte chunks are swizzled against LDS bank conflicts (gfx950: 64
// banks of 4 B; a 16-byte access is served 16 lanes per pass, so the 16 lanes
// of a lane group must meet 16 distinct 16-byte bank groups; measured with the
// bank-conflict counter):
//  * xoff (wide tiles of the scan): chunk q of row r lives at chunk
//    q ^ (r & 15).  A 16-byte read of one chunk by 16 consecutive rows (an
//    operand fragment) and a 16-byte store of a whole row by 16 lanes both
//    meet every bank group once.
//  * woff (wide tiles of the WY preparation, written 8 bytes at a time):
//    chunk q of row r lives at chunk q ^ (r & 7) ^ (q >> 3 & 1), which keeps
//    8-byte stores of the even, then the odd chunks of one row on distinct
//    banks.
//  * noff (narrow tiles): chunk q of row r lives at chunk q ^ (r >> 1 & 7);
//    two consecutive rows span the 64 banks, and a read of one chunk by 16
//    consecutive rows meets every bank group once.
__device__ __forceinline__ int xoff(int r, int q) { return r * 256 + ((q ^ (r & 15)) << 4); }
__device__ __forceinline__ int woff(int r, int q) { return r * 256 + ((q ^ (r & 7) ^ ((q >> 3) & 1)) << 4); }
__device__ __forceinline__ int noff(int r, int q) { return r * 128 + ((q ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ bf16x8 ldv(const bf16 *base, int byte_off) {
    return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(base) + byte_off);
}
__device__ __forceinline__ void stv(bf16 *base, int byte_off, const bf16x8 &v) {
    *reinterpret_cast<bf16x8 *>(reinterpret_cast<char *>(base) + byte_off) = v;
}

// Whole rows of a 64 x 128 bf16 chunk tile: lane l of load m covers row
// 4m + l/16, elements 8 (l % 16) .. +7 (16 B), so one instruction reads four
// full rows.
//
// Rows past the end of a ragged chunk are read as zeros: the loads go through
// a buffer resource whose range ends at the chunk's last valid row, and the
// hardware returns zeros for offsets beyond it (stores beyond it are dropped),
// so every load is unconditional and needs no clamping.  Zero rows are the
// padding of the MaxText PR, section "Implementation" (k = q = v = 0 with
// g = 0 and beta = 0 past the end): the columns of A0 diag(beta) vanish there,
// so T' has identity columns and, being lower triangular, no entries from
// such rows into valid rows; delta = diag(beta) T' R is zero on them, and
// their outputs are not stored.
//
// Loads go through a buffer resource whose base is row 0 of the chunk (wave
// uniform, in scalar registers) with a 32-bit per-lane byte offset, so a load
// needs one vector register for its address and no 64-bit vector arithmetic.
// The host guarantees that 64 rows of any tensor span less than 2 GiB.
constexpr uint32_t kRsrcWord3 = 0x00020000;   // gfx9 family: 32-bit raw data, no swizzle
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                             (int)kRsrcWord3);
}
// A resource covering nbytes from base: loads at offsets at or beyond nbytes
// return zeros and stores there are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void *base, uint32_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes, (int)kRsrcWord3);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint2 v) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{v.x, v.y}, r, voff, 0, 0);
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
__device__ __forceinline__ void load_rows(uint4 (&t)[16], const bf16 *base, uint32_t row_bytes,
                                          int L, int lane) {
    const __amdgpu_buffer_rsrc_t r = rsrc_n(base, (uint32_t)L * row_bytes);
    const uint32_t own = (uint32_t)(lane >> 4) * row_bytes + 16u * (lane & 15);
#pragma unroll
    for (int m = 0; m < 16; ++m) t[m] = bload16(r, own + (uint32_t)(4 * m) * row_bytes, 0);
}
// Store rows loaded by load_rows into a wide tile (xoff) in natural order: the 16 B
// of elements 8s .. 8s+7 are chunk s of the row, one 16-byte store per row
// and lane.
__device__ __forceinline__ void store_rows(bf16 *tile, const uint4 (&t)[16], int lane) {
    const int s = lane & 15;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int r = 4 * m + (lane >> 4);
        *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(tile) + xoff(r, s)) = t[m];
    }
}

// Inclusive prefix sum over the 64 lanes with DPP moves (no LDS round trips):
// shifts by 1, 2, 4, 8 within each row of 16 lanes (lanes whose source lies
// before the row start read 0), then lane 15 of rows 0 and 2 is added to rows
// 1 and 3, and lane 31 to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_mov0(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_cumsum(float x) {
    x += dpp_mov0<0x111, 0xf>(x);   // row_shr:1
    x += dpp_mov0<0x112, 0xf>(x);   // row_shr:2
    x += dpp_mov0<0x114, 0xf>(x);   // row_shr:4
    x += dpp_mov0<0x118, 0xf>(x);   // row_shr:8
    x += dpp_mov0<0x142, 0xa>(x);   // row_bcast:15 into rows 1, 3
    x += dpp_mov0<0x143, 0xc>(x);   // row_bcast:31 into rows 2, 3
    return x;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane 4a + b receives element b of the 8-byte runs addressed by lanes a,
// a + 4, a + 8, a + 12 of the group, in that order.
__device__ __forceinline__ bf16x4 ldtr(const bf16 *base, int byte_off) {
    typedef __attribute__((address_space(3))) short4v lds_short4v;
    const short4v x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4v *)(reinterpret_cast<const char *>(base) + byte_off));
    return __builtin_bit_cast(bf16x4, x);
}

// Gram tiles of one chunk (A0[r,s] = exp(G_r - G_s) k_r.k_s), from the k tile
// in MFMA operand layout: kt(c, kk) returns lane (i, g)'s operand for rows
// 16c + i, k-block kk (read k-block by k-block).  G2 is the cumulative
// log2-decay, Bv beta (both zero past the chunk end).  Blocks (a, b), b <= a,
// are numbered i = a (a + 1) / 2 + b; MASK selects the blocks formed (several
// waves can split them).  Writes, per lane, the off-diagonal blocks of
// -A0 diag(beta) (B layout, block (a, b) at ab[a (a - 1) / 2 + b]) and the raw
// diagonal blocks of k k^T (block (a, a) at ab[6 + a]).
template <int MASK = 0x3ff, class KT>
__device__ __forceinline__ void gram_to_ab(KT kt, const float *G2, const float *Bv, uint2 (*ab)[64], int lane) {
    const int li = lane & 15, lg = lane >> 4;
    // factors at rows 16t + 4g + e (B layout rows) and 16t + j (B layout column)
    f32x4 Gr4[4];
    float Gc[4], Bc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        Gr4[u] = *reinterpret_cast<const f32x4 *>(&G2[16 * u + 4 * lg]);
        Gc[u] = G2[16 * u + li];
        Bc[u] = Bv[16 * u + li];
    }
    // Gram k k^T: lane (j, g) element e of block (a, b) is k_{16a+4g+e} . k_{16b+j}.
    // Off-diagonal blocks leave negated, as -exp(G_r - G_s) k_r . k_s beta_s (the
    // sign of the block recursion of T' folded in), diagonal blocks raw.
    f32x4 acc[10];
#pragma unroll
    for (int i = 0; i < 10; ++i) acc[i] = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        bf16x8 kc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) kc[c] = kt(c, kk);
        int i = 0;
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
#pragma unroll
            for (int bb = 0; bb <= aa; ++bb, ++i)
                if ((MASK >> i) & 1) acc[i] = mma32(kc[aa], kc[bb], acc[i]);
    }
    int i = 0;
#pragma unroll
    for (int aa = 0; aa < 4; ++aa)
#pragma unroll
        for (int bb = 0; bb <= aa; ++bb, ++i) {
            if (!((MASK >> i) & 1)) continue;
            if (aa > bb) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = -Bc[bb] * ex2(Gr4[aa][e] - Gc[bb]) * acc[i][e];
                ab[aa * (aa - 1) / 2 + bb][lane] = __builtin_bit_cast(uint2, to4(v));
            } else {
                ab[6 + aa][lane] = __builtin_bit_cast(uint2, to4(acc[i]));
            }
        }
}

// Inverses of diagonal 16 x 16 blocks of T' = (I + A0 diag(beta))^{-1}, for
// the NBLK blocks listed in blk (compile-time constants), from the raw Gram
// blocks of gram_to_ab.  With N = (A0 diag(beta))_aa, strictly lower
// triangular, the inverse is built by recursive doubling of the block size:
// T_1 = I - N restricted to the 2 x 2 diagonal blocks (exact), then for
// l = 2, 4, 8, with B_l the part of N that joins two l x l diagonal blocks into
// one 2l x 2l block,
//   T_{2l} = T_l - T_l B_l T_l,
// which is the block formula [[A, 0], [B, D]]^{-1} = [[A^-1, 0],
// [-D^-1 B A^-1, D^-1]] applied to every 2l block at once.  Every product
// involves entries of the inverse itself, so nothing grows beyond it; the
// expansion (I - N)(I + N^2)(I + N^4)(I + N^8) does the same in exact
// arithmetic, but its powers of N reach binomial sizes (6435 for a key
// repeated over 16 tokens with beta = 1, g = 0), and rounding them to bf16
// loses the result.  T is kept in fp32 in both operand layouts (B layout TB:
// lane (j, g) holds T[4g+e][j]; A layout TA: lane (i, g) holds T[i][4g+e]):
//   W = B_l T (A = B_l, B = T);  T <- T - T W (A = T, B = W);
//   T^T <- T^T - W^T T^T (A = W^T, whose A layout is W's B layout; B = T^T,
//   whose B layout is T's A layout).
// Each level runs over all listed blocks before the next, so their dependent
// chains interleave.  Out: P[j] (bf16 B layout of T'_aa, which as an A
// operand is T'_aa^T) and Qf[j] (fp32 A layout of T'_aa).
// Per-lane 0/1 multipliers of diag_inverse (they depend on the lane only, so a
// caller that inverts many blocks forms them once).  For lane (i, g) and
// element e, x = 4g + e:
//   tb[e]   = 1 where B layout entry (x, i) lies in a 2 x 2 diagonal block below
//             the diagonal (x = i + 1, i even),
//   two[e]  = 1 where A layout entry (i, x) does (i = x + 1, x even),
//   lvl[l][e] = 1 where A layout entry (i, x), x < i, joins two 2^(l+1) blocks
//             into one 2^(l+2) block (the highest bit in which i and x differ
//             is bit l + 1),
//   eye[e]  = 1 on the diagonal (x = i).
struct InvMasks {
    f32x4 tb, two, eye, lvl[3];
};
__device__ __forceinline__ InvMasks inv_masks(int lane) {
    const int li = lane & 15, lg = lane >> 4;
    InvMasks m;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int x = 4 * lg + e;
        m.tb[e] = (x == li + 1 && !(li & 1)) ? 1.f : 0.f;
        m.two[e] = (li == x + 1 && !(x & 1)) ? 1.f : 0.f;
        m.eye[e] = x == li ? 1.f : 0.f;
#pragma unroll
        for (int l = 0; l < 3; ++l)
            m.lvl[l][e] = (x < li && (li >> (l + 2)) == (x >> (l + 2)) && (li >> (l + 1)) != (x >> (l + 1))) ? 1.f
                                                                                                               : 0.f;
    }
    return m;
}

// Inverses of diagonal 16 x 16 blocks of T' = (I + A0 diag(beta))^{-1}, for
// the NBLK blocks listed in blk (compile-time constants), from the raw Gram
// blocks of gram_to_ab.  With N = (A0 diag(beta))_aa, strictly lower
// triangular, the inverse is built by recursive doubling of the block size:
// T_1 = I - N restricted to the 2 x 2 diagonal blocks (exact), then for
// l = 2, 4, 8, with B_l the part of N that joins two l x l diagonal blocks into
// one 2l x 2l block,
//   T_{2l} = T_l - T_l B_l T_l,
// which is the block formula [[A, 0], [B, D]]^{-1} = [[A^-1, 0],
// [-D^-1 B A^-1, D^-1]] applied to every 2l block at once.  Every product
// involves entries of the inverse itself, so nothing grows beyond it; the
// expansion (I - N)(I + N^2)(I + N^4)(I + N^8) does the same in exact
// arithmetic, but its powers of N reach binomial sizes (6435 for a key
// repeated over 16 tokens with beta = 1, g = 0), and rounding them to bf16
// loses the result.  T is kept in fp32 in both operand layouts (B layout TB:
// lane (j, g) holds T[4g+e][j]; A layout TA: lane (i, g) holds T[i][4g+e]):
//   W' = -B_l T (A = -B_l, B = T);  T <- T + T W' (A = T, B = W');
//   T^T <- T^T + W'^T T^T (A = W'^T, whose A layout is W''s B layout; B = T^T,
//   whose B layout is T's A layout).
// Each level runs over all listed blocks before the next, so their dependent
// chains interleave.  Out: P[j] (bf16 B layout of T'_aa, which as an A
// operand is T'_aa^T) and Qf[j] (fp32 A layout of T'_aa).
template <int NBLK>
__device__ __forceinline__ void diag_inverse(const int (&blk)[NBLK], const uint2 (*ab)[64], const float *G2,
                                             const float *Bv, int lane, const InvMasks &m, bf16x4 (&P)[NBLK],
                                             f32x4 (&Qf)[NBLK]) {
    const int li = lane & 15, lg = lane >> 4;
    f32x4 TB[NBLK], TA[NBLK];
    bf16x4 BL[3][NBLK];   // A layout of -B_l, l = 2, 4, 8
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        const int aa = blk[j];
        const f32x4 Gr4 = *reinterpret_cast<const f32x4 *>(&G2[16 * aa + 4 * lg]);
        const f32x4 Br4 = *reinterpret_cast<const f32x4 *>(&Bv[16 * aa + 4 * lg]);
        const float Gc = G2[16 * aa + li], Bc = Bv[16 * aa + li];
        // raw k_{16a+4g+e} . k_{16a+j} (symmetric): B layout entry (r = 16a+4g+e,
        // s = 16a+j) if s < r, A layout entry (r' = 16a+j, s' = 16a+4g+e) if s' < r'
        const bf16x4 kk4 = __builtin_bit_cast(bf16x4, ab[6 + aa][lane]);
        f32x4 bl[3];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = 4 * lg + e;
            // exp(G_r - G_s) of the one layout entry that is kept (r > s), with
            // its sign, so that increasing decays (g > 0) stay exact
            const float kx = ex2(li < x ? Gr4[e] - Gc : Gc - Gr4[e]) * (float)kk4[e];
            // A layout entry N[i][x] (x < i, beta of column x); zero elsewhere
            const float va = x < li ? Br4[e] * kx : 0.f;
            TB[j][e] = __builtin_fmaf(-m.tb[e] * Bc, kx, m.eye[e]);
            TA[j][e] = __builtin_fmaf(-m.two[e], va, m.eye[e]);
#pragma unroll
            for (int l = 0; l < 3; ++l) bl[l][e] = -m.lvl[l][e] * va;
        }
#pragma unroll
        for (int l = 0; l < 3; ++l) BL[l][j] = to4(bl[l]);
    }
#pragma unroll
    for (int l = 0; l < 3; ++l) {
        f32x4 W[NBLK];
#pragma unroll
        for (int j = 0; j < NBLK; ++j) W[j] = mma16(BL[l][j], to4(TB[j]), zero4());
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const bf16x4 w = to4(W[j]);
            const bf16x4 ta = to4(TA[j]);
            TB[j] = mma16(ta, w, TB[j]);
            TA[j] = mma16(w, ta, TA[j]);
        }
    }
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
        P[j] = to4(TB[j]);
        Qf[j] = TA[j];
    }
}

// The off-diagonal blocks of T' by block forward substitution on T'^T, from
// the diagonal inverses (P, Qf of diag_inverse for blocks 0 .. 3) and the
// off-diagonal Gram tiles, then T' as row-major narrow tiles (the A operand
// layout of T' for a product over the chunk) in tb and, with tg non-null,
// T' diag(gamma), gamma_s = exp(G_s).  tg may share memory with ab: every read
// of ab comes first.
__device__ __forceinline__ void offdiag_store(const uint2 (*ab)[64], const float *G2, const bf16x4 (&P)[4],
                                              const f32x4 (&Qf)[4], bf16 *tb, bf16 *tg, int lane) {
    const int li = lane & 15, lg = lane >> 4;
    // AB[a][b] (a > b): B layout of -(A0 diag(beta))_ab
    bf16x4 AB[4][4];
    {
        const uint2 *abl = &ab[0][lane];
        AB[1][0] = __builtin_bit_cast(bf16x4, abl[0 * 64]);
        AB[2][0] = __builtin_bit_cast(bf16x4, abl[1 * 64]);
        AB[2][1] = __builtin_bit_cast(bf16x4, abl[2 * 64]);
        AB[3][0] = __builtin_bit_cast(bf16x4, abl[3 * 64]);
        AB[3][1] = __builtin_bit_cast(bf16x4, abl[4 * 64]);
        AB[3][2] = __builtin_bit_cast(bf16x4, abl[5 * 64]);
    }
    bf16x4 Q[4];
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) Q[aa] = to4(Qf[aa]);
    // off-diagonal blocks of T^T (B layout) = blocks of T (A layout):
    // U_ij = -(T'^T)_ii sum_{k=i+1..j} (A'^T)_ik (T'^T)_kj,  i < j
    // (the minus sign travels with AB)
    f32x4 U01, U12, U23, U02, U13, U03;
    {
        const f32x4 y01 = mma16(AB[1][0], Q[1], zero4());
        const f32x4 y12 = mma16(AB[2][1], Q[2], zero4());
        const f32x4 y23 = mma16(AB[3][2], Q[3], zero4());
        U01 = mma16(P[0], to4(y01), zero4());
        U12 = mma16(P[1], to4(y12), zero4());
        U23 = mma16(P[2], to4(y23), zero4());
        // terms that need no level-1 result first
        f32x4 y02 = mma16(AB[2][0], Q[2], zero4());
        f32x4 y13 = mma16(AB[3][1], Q[3], zero4());
        f32x4 y03 = mma16(AB[3][0], Q[3], zero4());
        y02 = mma16(AB[1][0], to4(U12), y02);
        y13 = mma16(AB[2][1], to4(U23), y13);
        y03 = mma16(AB[2][0], to4(U23), y03);
        U02 = mma16(P[0], to4(y02), zero4());
        U13 = mma16(P[1], to4(y13), zero4());
        y03 = mma16(AB[1][0], to4(U13), y03);
        U03 = mma16(P[0], to4(y03), zero4());
    }
    bf16x4 z4;
    z4[0] = z4[1] = z4[2] = z4[3] = (bf16)0.f;
    // keep every read of ab (and of whatever else shares memory with tb or tg)
    // above the writes
    asm volatile("" ::: "memory");
    stv(tb, noff(0 + li, 0 + lg), join(Q[0], z4));
    stv(tb, noff(16 + li, 0 + lg), join(to4(U01), Q[1]));
    stv(tb, noff(32 + li, 0 + lg), join(to4(U02), to4(U12)));
    stv(tb, noff(32 + li, 4 + lg), join(Q[2], z4));
    stv(tb, noff(48 + li, 0 + lg), join(to4(U03), to4(U13)));
    stv(tb, noff(48 + li, 4 + lg), join(to4(U23), Q[3]));
    if (tg) {
        // T' diag(gamma): element e of lane (i, g) in block (rb, cb) is column
        // 16 cb + 4g + e of T'
        f32x4 gm[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const f32x4 Gr4 = *reinterpret_cast<const f32x4 *>(&G2[16 * t + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) gm[t][e] = ex2(Gr4[e]);
        }
        auto sg = [&](const f32x4 &m, int cb) {
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) r[e] = m[e] * gm[cb][e];
            return to4(r);
        };
        stv(tg, noff(0 + li, 0 + lg), join(sg(Qf[0], 0), z4));
        stv(tg, noff(16 + li, 0 + lg), join(sg(U01, 0), sg(Qf[1], 1)));
        stv(tg, noff(32 + li, 0 + lg), join(sg(U02, 0), sg(U12, 1)));
        stv(tg, noff(32 + li, 4 + lg), join(sg(Qf[2], 2), z4));
        stv(tg, noff(48 + li, 0 + lg), join(sg(U03, 0), sg(U13, 1)));
        stv(tg, noff(48 + li, 4 + lg), join(sg(U23, 2), sg(Qf[3], 3)));
    }
}

// T' = (I + A0 diag(beta))^{-1} from the tiles of gram_to_ab, by one wave:
// the four diagonal inverses interleaved, then the off-diagonal blocks (see
// offdiag_store for tb and tg); m from inv_masks(lane).
__device__ __forceinline__ void invert_tprime(const uint2 (*ab)[64], const float *G2, const float *Bv,
                                              bf16 *tb, bf16 *tg, int lane, const InvMasks &m) {
    const int all[4] = {0, 1, 2, 3};
    bf16x4 P[4];
    f32x4 Qf[4];
    diag_inverse(all, ab, G2, Bv, lane, m, P, Qf);
    offdiag_store(ab, G2, P, Qf, tb, tg, lane);
}

}  // namespace mfma
}  // namespace gdn

#endif  // GDN_MFMA_TILE_H
