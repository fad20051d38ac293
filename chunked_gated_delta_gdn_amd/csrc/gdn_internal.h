// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

// Where every chain (one sequence segment) lives on the flattened token axis.
// Passed by value as a kernel argument.
//   batch mode:  sequence n owns tokens [n*seq_len, (n+1)*seq_len)
//   packed mode: sequence n owns tokens [seq_start[n], seq_start[n+1])
// Segment r of a sequence starts seg_start[r] tokens after the sequence start
// and ends at seg_start[r+1] (seg_start[n_seg] is a large sentinel clipped to
// the sequence end).  Chunks are counted per sequence: chunk j of sequence n
// starts at token start(n) + j*C and has global index chunk_base(n) + j.
struct ChainTable {
    int32_t n_seqs;
    int32_t n_seg;
    int32_t seq_len;     // batch mode: S; packed mode: 0
    int32_t packed;
    int32_t seq_start[GDN_MAX_SEQS + 1];
    int32_t chunk_start[GDN_MAX_SEQS + 1];
    int32_t seg_start[GDN_MAX_SEGMENTS + 1];
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

struct ScanArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    const void *wy_w, *wy_u;   // NULL: recompute in the kernel
    const float *h_in;
    void *o;
    float *h_out;
    float *M_out, *U_out;
    int32_t H;
    int32_t n_chains;
    ChainTable ct;
};

struct PrepArgs {
    const void *k, *v;
    const float *g, *beta;
    void *wy_w, *wy_u;
    int32_t H;
    int64_t n_chunks;
    ChainTable ct;
};

struct DecodeArgs {
    const void *q, *k, *v;
    const float *g, *beta;
    float *state;
    void *o;
    int32_t B, H;
};

struct ComposeArgs {
    const float *M, *U, *h0;
    float *h_in, *h_final;
    int32_t R, N, H;
};

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

bool shape_supported(int K, int V, int C);

}  // namespace gdn
