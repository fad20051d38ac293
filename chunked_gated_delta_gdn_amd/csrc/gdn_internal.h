// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// What a packed-mode scan launch does with one piece.
enum ItemKind : int {
    kItemEmit = 0,       // emit from h_in[piece]; the sequence's last piece writes h_out[sequence]
    kItemEmitFirst = 1,  // emit from h_in[sequence]; writes h_out[sequence]
    kItemCarry = 2,      // zero-state pass into M_out, U_out [piece]
};

// Where every chain (one sequence segment) lives on the flattened token axis.
// Passed by value as a kernel argument.
//   batch mode:  sequence n owns tokens [n*seq_len, (n+1)*seq_len)
//   packed mode: the chains are the pieces of the sequences (n_seg == 1):
//                piece p owns tokens [seq_start[p], seq_start[p+1]), and
//                n_seqs counts pieces
// Segment r of a sequence starts seg_start[r] tokens after the sequence start
// and ends at seg_start[r+1] (seg_start[n_seg] is a large sentinel clipped to
// the sequence end).  Chunks are counted per sequence: chunk j of sequence n
// starts at token start(n) + j*C and has global index chunk_base(n) + j.
// (Pieces start on chunk boundaries of their sequence, so a piece's chunk
// numbering is its sequence's.)
struct ChainTable {
    int32_t n_seqs;
    int32_t n_seg;
    int32_t seq_len;     // batch mode: S; packed mode: 0
    int32_t packed;
    int32_t seq_start[GDN_MAX_SEQS + 1];
    int32_t chunk_start[GDN_MAX_SEQS + 1];
    int32_t seg_start[GDN_MAX_SEGMENTS + 1];
    // packed mode: the launch's work items, longest first
    int32_t n_items;
    uint16_t item[GDN_MAX_SEQS];        // piece | ItemKind << 8
    uint8_t piece_seq[GDN_MAX_SEQS];    // sequence of each piece
    uint8_t piece_last[GDN_MAX_SEQS];   // 1 for the last piece of its sequence
};

struct ChainSpan {
    int64_t t0, t1;   // token range of the chain
    int64_t chunk0;   // global index of its first chunk
    int32_t seq, seg;
};

__host__ __device__ inline ChainSpan chain_span(const ChainTable &ct, int chain, int C) {
    ChainSpan s;
    s.seq = chain / ct.n_seg;
    s.seg = chain % ct.n_seg;
    int64_t a, b, cb;
    if (ct.packed) {
        a = ct.seq_start[s.seq];
        b = ct.seq_start[s.seq + 1];
        cb = ct.chunk_start[s.seq];
    } else {
        a = (int64_t)s.seq * ct.seq_len;
        b = a + ct.seq_len;
        cb = (int64_t)s.seq * ((ct.seq_len + C - 1) / C);
    }
    int64_t lo = a + ct.seg_start[s.seg];
    int64_t hi = a + ct.seg_start[s.seg + 1];
    s.t0 = lo < b ? lo : b;
    s.t1 = hi < b ? hi : b;
    s.chunk0 = cb + ct.seg_start[s.seg] / C;
    return s;
}

// One (chain, head) unit of a scan launch: its tokens and its state rows
// (row indices of [.., H, K, *] state arrays, head included).
struct UnitRef {
    ChainSpan sp;
    int64_t slot;       // emit: h_in row; carry: M_out / U_out row
    int64_t out_slot;   // emit: h_out row
    bool final_state;   // emit: writes h_out
    bool carry;
};

// Batch mode: chain = seq * n_seg + seg; h_in, M_out, U_out are [R, N, H].
__host__ __device__ inline UnitRef batch_unit(const ChainTable &ct, int chain, int h, int H, int C, bool carry) {
    UnitRef u;
    u.sp = chain_span(ct, chain, C);
    u.slot = ((int64_t)u.sp.seg * ct.n_seqs + u.sp.seq) * H + h;
    u.out_slot = (int64_t)u.sp.seq * H + h;
    u.final_state = u.sp.seg == ct.n_seg - 1;
    u.carry = carry;
    return u;
}

// Packed mode: item i of the launch.
__host__ __device__ inline UnitRef packed_unit(const ChainTable &ct, int i, int h, int H, int C) {
    const int code = ct.item[i];
    const int p = code & 0xff, kind = code >> 8;
    const int n = ct.piece_seq[p];
    UnitRef u;
    u.sp = chain_span(ct, p, C);
    u.slot = (int64_t)(kind == kItemEmitFirst ? n : p) * H + h;
    u.out_slot = (int64_t)n * H + h;
    u.final_state = kind == kItemEmitFirst || ct.piece_last[p] != 0;
    u.carry = kind == kItemCarry;
    return u;
}

struct ScanArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const void *wy_w, *wy_u;   // NULL: recompute in the kernel
    const float *h_in;
    void *o;
    float *h_out;
    float *M_out, *U_out;
    int32_t H;          // value heads (state heads)
    int32_t Hk;         // heads of q and k: value head h reads key head h / (H / Hk)
    int32_t n_chains;   // batch mode: chains; packed mode: ct.n_items
    ChainTable ct;
};
// kernel arguments stay within the 4 KiB the runtime passes
static_assert(sizeof(ScanArgs) + 64 <= 4096, "scan kernel arguments too large");

struct PrepArgs {
    const void *k, *v;
    const float *g, *beta;
    void *wy_w, *wy_u;
    int32_t H, Hk;      // value heads; heads of k (value head h reads key head h / (H / Hk))
    int64_t n_chunks;
    ChainTable ct;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float *state;
    void *o;
    int32_t B, H, Hk;   // value heads H; q, k have Hk heads (value head h reads key head h / (H / Hk))
};

struct ComposeArgs {
    const float *M, *U, *h0;
    float *h_in, *h_final;
    int32_t R, N, H;
    // packed mode: sequence n's pieces are seq_first[n] .. seq_first[n+1]-1;
    // the scan starts at piece `first` of each; state rows are [P, H]
    int32_t packed, first;
    // 1: walk the steps last to first (the reverse scan of the backward pass,
    // with M holding the transposed maps)
    int32_t reverse;
    int16_t seq_first[GDN_MAX_SEQS + 1];
};

// Depthwise causal convolution: x, y [T, D]; weight [D, W]; states [N, D, W-1].
struct ConvArgs {
    const void *x, *weight, *state_in;
    void *state_out, *y;
    int64_t T;                 // tokens
    int32_t D, W;              // channels, taps
    int32_t S, N, packed;      // batch: N sequences of S tokens; packed: offsets in start
    int32_t activation;        // 0: none, 1: SiLU
    int32_t start[GDN_MAX_SEQS + 1];
    // the 8-channel kernels' token runs, laid out per sequence (set by their launcher)
    int64_t n_blocks;
    int32_t n_cg;              // channel groups (workgroups per run)
    int32_t block_start[GDN_MAX_SEQS + 1];
};

// Gated RMSNorm over rows of V: y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z).
struct NormArgs {
    const void *o, *z;         // z nullable (no gate)
    const float *weight;       // [V]
    void *y;
    int64_t rows;
    int32_t V;
    float eps;
};

// Backward pass.  Gradients in the layouts of their inputs; the fp32
// workspace holds, per (chunk, head): T = (I + A)^{-1}, attn and the decayed
// Gram Dec (.) K K^T (C x C each), w (C x K), u, delta, ddelta (C x V), and
// the state and its gradient at the chunk's start and end (K x V at K = V =
// 128, else transposed V x K).
struct BwdArgs {
    const void *q, *k, *v, *dout;
    const float *g, *beta, *h0, *dhT;
    void *dq, *dk, *dv;
    float *dg, *dbeta, *dh0;
    float *T, *attn, *Ak, *w, *u, *hs, *dhs, *d, *dd;
    float *dq_acc, *dk_acc;   // grouped key heads: per value head dq, dk [T, H, K]; else NULL
    // Chains that split a sequence (segments, pieces), state rows [slots, H]
    // (slot as in ComposeArgs): a chain that does not start its sequence
    // starts from h_in, one that does not end it from dh_in (NULL when every
    // chain is a whole sequence).  Carry launches write, per chain of a split
    // sequence, the affine map of the forward scan (M [K,K] and its transpose
    // Mt for every chain; U [K,V] for all but the last) and the reverse
    // scan's offset E [K,V] for all but the first (the gradient at the
    // chain's start given a zero gradient at its end).
    const float *h_in, *dh_in;
    float *M, *Mt, *U, *E;
    int32_t carry;
    int32_t n_units;          // (chain, head) units of a state-scan launch (set by its launcher)
    int32_t N;                // sequences
    int32_t H, Hk;            // value heads; heads of q and k (value head h reads key head h / (H / Hk))
    int64_t n_chunks, tokens; // chunks over all sequences; tokens
    ChainTable ct;
};

// Where chain `chain` sits in its sequence.
struct ChainPos {
    int64_t slot;   // state row / H of the chain's boundary states and carries
    int32_t seq;
    bool first, last;
};
__host__ __device__ inline ChainPos chain_pos(const ChainTable &ct, int chain, int N) {
    ChainPos c;
    if (ct.packed) {
        c.seq = ct.piece_seq[chain];
        c.slot = chain;
        c.first = chain == 0 || ct.piece_seq[chain - 1] != ct.piece_seq[chain];
        c.last = ct.piece_last[chain] != 0;
    } else {
        const int seg = chain % ct.n_seg;
        c.seq = chain / ct.n_seg;
        c.slot = (int64_t)seg * N + c.seq;
        c.first = seg == 0;
        c.last = seg == ct.n_seg - 1;
    }
    return c;
}
static_assert(sizeof(BwdArgs) + 64 <= 4096, "backward kernel arguments too large");

// Launchers (return the hipError_t of the launch).
hipError_t launch_scan(int K, int V, int C, int dtype, bool carry, const ScanArgs &a,
                       hipStream_t s);
// segment 0 of every sequence emitted (h_in, o, h_out), segments 1 .. R-1 carried
hipError_t launch_scan_head(int K, int V, int C, int dtype, const ScanArgs &a, const float *h_in, void *o,
                            float *h_out, hipStream_t s);
hipError_t launch_prepare(int K, int V, int C, int dtype, const PrepArgs &a, hipStream_t s);
bool mfma_prepare_available(int K, int V, int C, int dtype);
hipError_t launch_prepare_mfma(const PrepArgs &a, hipStream_t s);
hipError_t launch_decode(int K, int V, int dtype, const DecodeArgs &a, hipStream_t s);
hipError_t launch_compose(int K, int V, const ComposeArgs &a, hipStream_t s);
hipError_t launch_causal_conv(int dtype, const ConvArgs &a, hipStream_t s);
hipError_t launch_gated_rmsnorm(int dtype, const NormArgs &a, hipStream_t s);
// the backward launches; n_chains = chains (sequences, or their segments or
// pieces); when chains split sequences, fwd and rev describe the compose
// launches between the carry and emit scans (else both NULL)
hipError_t launch_backward(int K, int V, int C, int dtype, const BwdArgs &a, int n_chains,
                           const ComposeArgs *fwd, const ComposeArgs *rev, hipStream_t s);

bool shape_supported(int K, int V, int C);

}  // namespace gdn
