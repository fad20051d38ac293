// Host side of the C ABI declared in include/gdn.h: argument validation,
// chain tables, workspace sizing and kernel dispatch.  Every check runs
// before the first launch, so a failing call writes nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "gdn_internal.h"

namespace gdn {
hipError_t launch_scan_generic(int K, int V, int C, int dtype, bool carry, const ScanArgs &a,
                               hipStream_t s);
hipError_t launch_scan_mfma(int K, int V, int C, int dtype, bool carry, const ScanArgs &a,
                            hipStream_t s, bool *handled);
hipError_t launch_scan_head_mfma(int K, int V, int C, int dtype, const ScanArgs &a, const float *h_in, void *o,
                                 float *h_out, hipStream_t s, bool *handled);
bool mfma_scan_available(int K, int V, int C, int dtype);

bool shape_supported(int K, int V, int C) {
    return (K == 32 && V == 32 && C == 16) || (K == 128 && V == 128 && C == 64);
}

hipError_t launch_scan(int K, int V, int C, int dtype, bool carry, const ScanArgs &a,
                       hipStream_t s) {
    bool handled = false;
    hipError_t e = launch_scan_mfma(K, V, C, dtype, carry, a, s, &handled);
    if (handled) return e;
    return launch_scan_generic(K, V, C, dtype, carry, a, s);
}

hipError_t launch_scan_head(int K, int V, int C, int dtype, const ScanArgs &a, const float *h_in, void *o,
                            float *h_out, hipStream_t s) {
    bool handled = false;
    hipError_t e = launch_scan_head_mfma(K, V, C, dtype, a, h_in, o, h_out, s, &handled);
    if (handled) return e;
    if (a.ct.packed) {
        // two launches over the emitting and the carrying items
        ScanArgs e_args = a, c_args = a;
        e_args.ct.n_items = c_args.ct.n_items = 0;
        for (int i = 0; i < a.ct.n_items; ++i) {
            ScanArgs &dst = (a.ct.item[i] >> 8) == kItemCarry ? c_args : e_args;
            dst.ct.item[dst.ct.n_items++] = a.ct.item[i];
        }
        e_args.n_chains = e_args.ct.n_items;
        c_args.n_chains = c_args.ct.n_items;
        if (e_args.n_chains > 0) {
            e = launch_scan_generic(K, V, C, dtype, false, e_args, s);
            if (e != hipSuccess) return e;
        }
        return c_args.n_chains > 0 ? launch_scan_generic(K, V, C, dtype, true, c_args, s) : hipSuccess;
    }
    // two launches: the head segments emitted, then the others carried, each over
    // a chain table restricted to its segments (token offsets stay absolute)
    const int R = a.ct.n_seg;
    ScanArgs e_args = a;
    e_args.ct.n_seg = 1;
    e_args.ct.seg_start[1] = a.ct.seg_start[1];
    e_args.n_chains = a.ct.n_seqs;
    e_args.h_in = h_in;
    e_args.o = o;
    e_args.h_out = h_out;
    e_args.M_out = e_args.U_out = nullptr;
    e = launch_scan_generic(K, V, C, dtype, false, e_args, s);
    if (e != hipSuccess) return e;
    ScanArgs c_args = a;
    c_args.ct.n_seg = R - 1;
    for (int r = 0; r < R; ++r) c_args.ct.seg_start[r] = a.ct.seg_start[r + 1];
    c_args.n_chains = a.ct.n_seqs * (R - 1);
    return launch_scan_generic(K, V, C, dtype, true, c_args, s);
}
}  // namespace gdn

using namespace gdn;

namespace {

thread_local char g_err[512] = "";

gdn_status fail(gdn_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Resolved {
    int N = 0;            // sequences (B or n_seqs)
    int R = 1;            // segments per sequence (batch mode)
    int P = 0;            // pieces (packed mode), N * R (batch mode)
    int64_t T = 0;        // tokens on the flattened axis
    int64_t n_chunks = 0; // chunks over all sequences
    int16_t seq_first[GDN_MAX_SEQS + 1];   // packed mode: first piece of each sequence
    ChainTable ct;
};

gdn_status resolve(const gdn_problem *p, Resolved &out) {
    if (!p) return fail(GDN_EINVAL, "problem descriptor is NULL");
    if (p->B < 1 || p->S < 0 || p->H < 1 || p->K < 1 || p->V < 1 || p->C < 1)
        return fail(GDN_EINVAL, "bad sizes B=%d S=%d H=%d K=%d V=%d C=%d", p->B, p->S, p->H,
                    p->K, p->V, p->C);
    if (!shape_supported(p->K, p->V, p->C))
        return fail(GDN_EUNSUPPORTED, "(K,V,C)=(%d,%d,%d) not built; supported (32,32,16), "
                                      "(128,128,64)", p->K, p->V, p->C);
    if (p->dtype != GDN_F32 && p->dtype != GDN_BF16)
        return fail(GDN_EUNSUPPORTED, "dtype %d not supported", p->dtype);
    if (p->n_seqs < 0) return fail(GDN_EINVAL, "n_seqs %d < 0", p->n_seqs);
    if (p->H_qk < 0 || p->H_qk > p->H || (p->H_qk > 0 && p->H % p->H_qk != 0))
        return fail(GDN_EINVAL, "H_qk = %d must divide H = %d (0 means H)", p->H_qk, p->H);
    if (p->max_piece_chunks < 0) return fail(GDN_EINVAL, "max_piece_chunks %d < 0", p->max_piece_chunks);
    if (p->n_seqs == 0 && p->max_piece_chunks != 0)
        return fail(GDN_EINVAL, "max_piece_chunks applies to packed problems only (use segments)");
    memset(&out.ct, 0, sizeof(out.ct));
    const int C = p->C;
    if (p->n_seqs > 0) {
        if (p->B != 1) return fail(GDN_EINVAL, "packed mode needs B == 1 (got %d)", p->B);
        if (p->n_seqs > GDN_MAX_SEQS)
            return fail(GDN_EUNSUPPORTED, "%d sequences > GDN_MAX_SEQS", p->n_seqs);
        if (!p->cu_seqlens) return fail(GDN_EINVAL, "cu_seqlens is NULL in packed mode");
        if (p->n_segments != 1)
            return fail(GDN_EUNSUPPORTED, "segments are not supported in packed mode (use max_piece_chunks)");
        const int32_t *cu = p->cu_seqlens;
        if (cu[0] != 0) return fail(GDN_EORDER, "cu_seqlens[0] = %d, must be 0", cu[0]);
        for (int n = 0; n < p->n_seqs; ++n)
            if (cu[n + 1] < cu[n])
                return fail(GDN_EORDER, "cu_seqlens decreases at %d (%d -> %d)", n, cu[n],
                            cu[n + 1]);
        if (cu[p->n_seqs] != p->S)
            return fail(GDN_EINVAL, "cu_seqlens[n_seqs] = %d != S = %d", cu[p->n_seqs], p->S);
        // the chains are the pieces: a sequence of nc > m chunks becomes
        // R_n = ceil(nc / m) pieces, piece s starting at chunk s * nc / R_n
        const int64_t m = p->max_piece_chunks;
        int64_t chunks = 0;
        int P = 0;
        for (int n = 0; n < p->n_seqs; ++n) {
            const int64_t nc = cdiv(cu[n + 1] - cu[n], C);
            const int64_t Rn = (m > 0 && nc > m) ? cdiv(nc, m) : 1;
            if (P + Rn > GDN_MAX_SEQS)
                return fail(GDN_EUNSUPPORTED, "more than GDN_MAX_SEQS = %d pieces (max_piece_chunks %d)",
                            GDN_MAX_SEQS, p->max_piece_chunks);
            out.seq_first[n] = (int16_t)P;
            for (int64_t sgm = 0; sgm < Rn; ++sgm) {
                const int64_t c0 = sgm * nc / Rn;
                out.ct.seq_start[P] = (int32_t)(cu[n] + c0 * C);
                out.ct.chunk_start[P] = (int32_t)(chunks + c0);
                out.ct.piece_seq[P] = (uint8_t)n;
                out.ct.piece_last[P] = sgm == Rn - 1;
                ++P;
            }
            chunks += nc;
        }
        out.seq_first[p->n_seqs] = (int16_t)P;
        out.ct.seq_start[P] = cu[p->n_seqs];
        out.ct.chunk_start[P] = (int32_t)chunks;
        out.ct.packed = 1;
        out.ct.n_seqs = P;
        out.ct.n_seg = 1;
        out.ct.seg_start[0] = 0;
        out.ct.seg_start[1] = 0x3fffffff;
        out.N = p->n_seqs;
        out.R = 1;
        out.P = P;
        out.n_chunks = chunks;
    } else {
        const int R = p->n_segments;
        if (R < 1) return fail(GDN_EINVAL, "n_segments %d < 1", R);
        if (R > GDN_MAX_SEGMENTS)
            return fail(GDN_EUNSUPPORTED, "%d segments > GDN_MAX_SEGMENTS", R);
        const int64_t nc = cdiv(p->S, C);
        if (R > 1 && R > nc)
            return fail(GDN_EINVAL, "%d segments but only %lld chunks", R, (long long)nc);
        if (p->seg_starts) {
            const int32_t *ss = p->seg_starts;
            if (ss[0] != 0) return fail(GDN_EORDER, "seg_starts[0] = %d, must be 0", ss[0]);
            for (int r = 0; r < R; ++r) {
                if (ss[r] % C != 0)
                    return fail(GDN_EORDER, "seg_starts[%d] = %d is not a multiple of C = %d", r,
                                ss[r], C);
                if (r > 0 && ss[r] <= ss[r - 1])
                    return fail(GDN_EORDER, "segments must be contiguous and in order: "
                                            "seg_starts[%d] = %d <= seg_starts[%d] = %d",
                                r, ss[r], r - 1, ss[r - 1]);
                if (R > 1 && ss[r] >= p->S)
                    return fail(GDN_EORDER, "seg_starts[%d] = %d >= S = %d", r, ss[r], p->S);
                out.ct.seg_start[r] = ss[r];
            }
        } else {
            for (int r = 0; r < R; ++r) out.ct.seg_start[r] = (int32_t)((r * nc / R) * C);
        }
        out.ct.seg_start[R] = p->S;
        out.ct.packed = 0;
        out.ct.n_seqs = p->B;
        out.ct.seq_len = p->S;
        out.ct.n_seg = R;
        out.N = p->B;
        out.R = R;
        out.P = p->B * R;
        out.n_chunks = (int64_t)p->B * nc;
    }
    out.T = p->n_seqs > 0 ? (int64_t)p->S : (int64_t)p->B * p->S;
    const int64_t wgs = (int64_t)out.P * p->H * (p->K + p->V);
    if (wgs > 0x7fffffffLL || out.n_chunks * p->H > 0x7fffffffLL)
        return fail(GDN_EUNSUPPORTED, "problem too large for one launch");
    // The kernels address the rows of one chunk through a buffer resource at the
    // chunk's first row with 32-bit byte offsets (and 2^31 - 1 records), so C rows
    // of q, k (H_qk heads) and of v, o (H heads) must span less than 2 GiB.
    {
        const int64_t es = p->dtype == GDN_F32 ? 4 : 2;
        const int64_t Hk = p->H_qk > 0 ? p->H_qk : p->H;
        const int64_t span = (int64_t)C * std::max(Hk * p->K, (int64_t)p->H * p->V) * es;
        if (span >= 0x80000000LL || (int64_t)C * p->H * 4 >= 0x80000000LL)
            return fail(GDN_EUNSUPPORTED, "%d token rows of the inputs span %lld bytes, at or above the "
                                          "2 GiB a chunk may span", C, (long long)span);
    }
    return GDN_OK;
}

size_t elem_size(int dtype) { return dtype == GDN_F32 ? 4 : 2; }

gdn_status check_ptr(const void *ptr, const char *name, bool required) {
    if (!ptr) return required ? fail(GDN_EINVAL, "%s is NULL", name) : GDN_OK;
    if (!aligned16(ptr)) return fail(GDN_EINVAL, "%s is not 16-byte aligned", name);
    return GDN_OK;
}

#define GDN_TRY(expr)                      \
    do {                                   \
        gdn_status _st = (expr);           \
        if (_st != GDN_OK) return _st;     \
    } while (0)

gdn_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(GDN_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
    return GDN_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b) return false;
    const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

// Packed mode: the work items of a gdn_scan launch in r.ct.item, longest piece
// first (so that the longest chains are dispatched first).  Counts the
// emitting and carrying items.
void packed_items(Resolved &r, int32_t mode, int &n_emit, int &n_carry) {
    ChainTable &ct = r.ct;
    n_emit = n_carry = 0;
    int n = 0;
    for (int p = 0; p < r.P; ++p) {
        const bool first = p == r.seq_first[ct.piece_seq[p]];
        int kind;
        if (mode == GDN_SCAN_EMIT) kind = kItemEmit;
        else if (mode == GDN_SCAN_CARRY) kind = kItemCarry;
        else if (mode == GDN_SCAN_HEAD_EMIT_CARRY) kind = first ? kItemEmitFirst : ct.piece_last[p] ? -1 : kItemCarry;
        else kind = first ? -1 : kItemEmit;   // GDN_SCAN_TAIL_EMIT
        if (kind < 0) continue;
        ct.item[n++] = (uint16_t)(p | kind << 8);
        if (kind == kItemCarry) ++n_carry;
        else ++n_emit;
    }
    ct.n_items = n;
    std::stable_sort(ct.item, ct.item + n, [&](uint16_t x, uint16_t y) {
        const int px = x & 0xff, py = y & 0xff;
        return ct.chunk_start[px + 1] - ct.chunk_start[px] > ct.chunk_start[py + 1] - ct.chunk_start[py];
    });
}

}  // namespace

extern "C" {

gdn_status gdn_validate(const gdn_problem *p) {
    g_err[0] = 0;
    Resolved r;
    return resolve(p, r);
}

int32_t gdn_num_pieces(const gdn_problem *p) {
    Resolved r;
    if (resolve(p, r) != GDN_OK) return -1;
    return r.P;
}

size_t gdn_wy_workspace_bytes(const gdn_problem *p) {
    Resolved r;
    if (resolve(p, r) != GDN_OK) return 0;
    return (size_t)r.n_chunks * p->H * p->C * (p->K + p->V) * elem_size(p->dtype);
}

// A WY workspace given to gdn_chunk_prepare or gdn_scan must hold the whole
// problem's factors.
static gdn_status check_wy(const gdn_problem *p, const Resolved &r, const void *wy, size_t wy_bytes) {
    if (!wy) return GDN_OK;
    const size_t need = (size_t)r.n_chunks * p->H * p->C * (p->K + p->V) * elem_size(p->dtype);
    if (wy_bytes < need)
        return fail(GDN_EWORKSPACE, "WY workspace of %zu bytes, the problem needs %zu", wy_bytes, need);
    return GDN_OK;
}

size_t gdn_segment_workspace_bytes(const gdn_problem *p) {
    Resolved r;
    if (resolve(p, r) != GDN_OK) return 0;
    return (size_t)r.P * p->H * p->K * (size_t)(p->K + p->V) * sizeof(float);
}

gdn_status gdn_chunk_prepare(const gdn_problem *p, const void *k, const void *v,
                             const float *g, const float *beta, void *wy, size_t wy_bytes, void *stream) {
    g_err[0] = 0;
    Resolved r;
    GDN_TRY(resolve(p, r));
    const bool any = r.T > 0;
    GDN_TRY(check_ptr(k, "k", any));
    GDN_TRY(check_ptr(v, "v", any));
    GDN_TRY(check_ptr(g, "g", any));
    GDN_TRY(check_ptr(beta, "beta", any));
    GDN_TRY(check_ptr(wy, "wy", r.n_chunks > 0));
    GDN_TRY(check_wy(p, r, wy, wy_bytes));
    if (r.n_chunks == 0) return GDN_OK;
    PrepArgs a;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.wy_w = wy;
    a.wy_u = static_cast<char *>(wy) + (size_t)r.n_chunks * p->H * p->C * p->K * elem_size(p->dtype);
    a.H = p->H;
    a.Hk = p->H_qk > 0 ? p->H_qk : p->H;
    a.n_chunks = r.n_chunks;
    a.ct = r.ct;
    (void)hipGetLastError();
    return launched(launch_prepare(p->K, p->V, p->C, p->dtype, a, (hipStream_t)stream),
                    "gdn_chunk_prepare");
}

// GDN_SCAN_HEAD_EMIT_CARRY: segment 0 (first piece) of every sequence emitted, the
// others carried, in one launch on the matrix-core path.
static gdn_status scan_head(const gdn_problem *p, Resolved &r, const void *q, const void *k, const void *v,
                            const float *g, const float *beta, const void *wy, size_t wy_bytes,
                            const float *h_in, void *o,
                            float *h_out, float *M_out, float *U_out, void *stream) {
    if (!r.ct.packed && r.R < 2)
        return fail(GDN_EINVAL, "GDN_SCAN_HEAD_EMIT_CARRY needs n_segments >= 2 in batch mode (got %d)", r.R);
    int n_emit = 0, n_carry = 1;
    if (r.ct.packed) packed_items(r, GDN_SCAN_HEAD_EMIT_CARRY, n_emit, n_carry);
    const bool any = r.T > 0;
    GDN_TRY(check_ptr(q, "q", any));
    GDN_TRY(check_ptr(k, "k", any));
    GDN_TRY(check_ptr(v, "v", any));
    GDN_TRY(check_ptr(g, "g", any));
    GDN_TRY(check_ptr(beta, "beta", any));
    GDN_TRY(check_ptr(wy, "wy", false));
    GDN_TRY(check_wy(p, r, wy, wy_bytes));
    GDN_TRY(check_ptr(o, "o", any));
    GDN_TRY(check_ptr(h_in, "h_in", false));
    GDN_TRY(check_ptr(h_out, "h_out", false));
    GDN_TRY(check_ptr(M_out, "M_out", n_carry > 0));
    GDN_TRY(check_ptr(U_out, "U_out", n_carry > 0));
    ScanArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.wy_w = wy;
    a.wy_u = wy ? static_cast<const char *>(wy) + (size_t)r.n_chunks * p->H * p->C * p->K * elem_size(p->dtype)
                : nullptr;
    a.h_in = nullptr;
    a.o = nullptr;
    a.h_out = nullptr;
    a.M_out = M_out;
    a.U_out = U_out;
    a.H = p->H;
    a.Hk = p->H_qk > 0 ? p->H_qk : p->H;
    a.n_chains = r.N * (r.R - 1);
    a.ct = r.ct;
    if (r.ct.packed) {
        // the items say which pieces emit and which carry; every pointer rides in a
        a.h_in = h_in;
        a.o = o;
        a.h_out = h_out;
        a.n_chains = r.ct.n_items;
        if (a.n_chains == 0) return GDN_OK;
    }
    (void)hipGetLastError();
    return launched(launch_scan_head(p->K, p->V, p->C, p->dtype, a, h_in, o, h_out, (hipStream_t)stream),
                    "gdn_scan");
}

gdn_status gdn_scan(const gdn_problem *p, int32_t mode, const void *q, const void *k,
                    const void *v, const float *g, const float *beta, const void *wy, size_t wy_bytes,
                    const float *h_in, void *o, float *h_out, float *M_out, float *U_out,
                    void *stream) {
    g_err[0] = 0;
    Resolved r;
    GDN_TRY(resolve(p, r));
    if (mode != GDN_SCAN_EMIT && mode != GDN_SCAN_CARRY && mode != GDN_SCAN_HEAD_EMIT_CARRY &&
        mode != GDN_SCAN_TAIL_EMIT)
        return fail(GDN_EINVAL, "unknown scan mode %d", mode);
    if (mode == GDN_SCAN_HEAD_EMIT_CARRY)
        return scan_head(p, r, q, k, v, g, beta, wy, wy_bytes, h_in, o, h_out, M_out, U_out, stream);
    if (mode == GDN_SCAN_TAIL_EMIT && !r.ct.packed)
        return fail(GDN_EINVAL, "GDN_SCAN_TAIL_EMIT needs a packed problem (batch callers slice the tensors)");
    const bool carry = mode == GDN_SCAN_CARRY;
    int n_emit = 0, n_carry = 0;
    if (r.ct.packed) packed_items(r, mode, n_emit, n_carry);
    const bool any = r.T > 0;
    GDN_TRY(check_ptr(k, "k", any));
    GDN_TRY(check_ptr(v, "v", any));
    GDN_TRY(check_ptr(g, "g", any));
    GDN_TRY(check_ptr(beta, "beta", any));
    GDN_TRY(check_ptr(wy, "wy", false));
    GDN_TRY(check_wy(p, r, wy, wy_bytes));
    if (carry) {
        GDN_TRY(check_ptr(M_out, "M_out", true));
        GDN_TRY(check_ptr(U_out, "U_out", true));
    } else {
        GDN_TRY(check_ptr(q, "q", any));
        GDN_TRY(check_ptr(o, "o", any));
        GDN_TRY(check_ptr(h_in, "h_in", false));
        GDN_TRY(check_ptr(h_out, "h_out", false));
        // h_in rows: [R, N] segments (batch) or [P] pieces (packed)
        if (h_out && h_in && r.P > r.N) {
            const size_t state = (size_t)p->H * p->K * p->V * sizeof(float);
            if (overlaps(h_in, state * r.P, h_out, state * r.N))
                return fail(GDN_EINVAL, "h_out may alias h_in only with one segment (piece) per sequence");
        }
    }
    ScanArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.wy_w = wy;
    a.wy_u = wy ? static_cast<const char *>(wy) +
                      (size_t)r.n_chunks * p->H * p->C * p->K * elem_size(p->dtype)
                : nullptr;
    a.h_in = carry ? nullptr : h_in;
    a.o = carry ? nullptr : o;
    a.h_out = carry ? nullptr : h_out;
    a.M_out = carry ? M_out : nullptr;
    a.U_out = carry ? U_out : nullptr;
    a.H = p->H;
    a.Hk = p->H_qk > 0 ? p->H_qk : p->H;
    a.n_chains = r.ct.packed ? r.ct.n_items : r.N * r.R;
    a.ct = r.ct;
    if (a.n_chains == 0) return GDN_OK;
    (void)hipGetLastError();
    return launched(launch_scan(p->K, p->V, p->C, p->dtype, carry, a, (hipStream_t)stream),
                    "gdn_scan");
}

// ---- gdn_forward: the whole forward in one call ----------------------------------------

// Byte offsets of gdn_forward's workspace (fp32 state rows; every region a
// multiple of H*K*V*4 bytes, so 16-byte aligned when the base is):
//   batch, R >= 2:  h1 [N,H,K,V] | M [R-2,N,H,K,K] | U [R-2,N,H,K,V] | h_all [R-1,N,H,K,V]
//   packed, P > N:  hs [N,H,K,V] | M [P,H,K,K]     | U [P,H,K,V]     | h_in [P,H,K,V]
// Problems whose sequences are one chain each need none (total = 0).
struct FwdLayout {
    size_t h1 = 0, M = 0, U = 0, hin = 0, total = 0;
};

static FwdLayout forward_layout(const gdn_problem *p, const Resolved &r) {
    FwdLayout L;
    const size_t sk = (size_t)p->H * p->K * p->K * sizeof(float);
    const size_t sv = (size_t)p->H * p->K * p->V * sizeof(float);
    size_t nm, nh;   // state rows of M and U; of h_all / h_in
    if (!r.ct.packed) {
        if (r.R < 2) return L;
        nm = (size_t)(r.R - 2) * r.N;
        nh = (size_t)(r.R - 1) * r.N;
    } else {
        if (r.P == r.N) return L;
        nm = nh = (size_t)r.P;
    }
    L.M = (size_t)r.N * sv;
    L.U = L.M + nm * sk;
    L.hin = L.U + nm * sv;
    L.total = L.hin + nh * sv;
    return L;
}

// The schedule of gdn_forward (the segment pass of the MaxText PR, section
// "Implementation", without its redundant work), on the stream, with the
// workspace at ws (FwdLayout).  Arguments are already validated.
static gdn_status forward_run(const gdn_problem *p, Resolved &r, const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const float *h0, void *o, float *h_out,
                              char *ws, hipStream_t s, const char *who) {
    ScanArgs a;
    memset(&a, 0, sizeof(a));
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.wy_w = a.wy_u = nullptr;
    a.H = p->H;
    a.Hk = p->H_qk > 0 ? p->H_qk : p->H;
    const int K = p->K, V = p->V, C = p->C, dt = p->dtype;
    const FwdLayout L = forward_layout(p, r);
    (void)hipGetLastError();
    if (L.total == 0) {
        // one chain per sequence: the emitting scan alone
        a.h_in = h0;
        a.o = o;
        a.h_out = h_out;
        if (r.ct.packed) {
            int ne, nc;
            packed_items(r, GDN_SCAN_EMIT, ne, nc);
            a.n_chains = r.ct.n_items;
        } else {
            a.n_chains = r.N * r.R;
        }
        a.ct = r.ct;
        if (a.n_chains == 0) return GDN_OK;
        return launched(launch_scan(K, V, C, dt, false, a, s), who);
    }
    float *h1 = reinterpret_cast<float *>(ws + L.h1);
    float *M = reinterpret_cast<float *>(ws + L.M);
    float *U = reinterpret_cast<float *>(ws + L.U);
    float *hin = reinterpret_cast<float *>(ws + L.hin);
    if (!r.ct.packed) {
        const int R = r.R, N = r.N;
        // 1. segment 0 emitted from h0, its final state (the state entering
        //    segment 1) to h1; segments 1 .. R-2 carried into M, U.  The chain
        //    table stops at the start of segment R-1.
        ScanArgs hd = a;
        hd.ct = r.ct;
        hd.ct.n_seg = R - 1;
        if (R == 2) {
            hd.h_in = h0;
            hd.o = o;
            hd.h_out = h1;
            hd.n_chains = N;
            GDN_TRY(launched(launch_scan(K, V, C, dt, false, hd, s), who));
        } else {
            hd.M_out = M;
            hd.U_out = U;
            hd.n_chains = N * (R - 2);
            GDN_TRY(launched(launch_scan_head(K, V, C, dt, hd, h0, o, h1, s), who));
            // 2. the states entering segments 1 .. R-1: h_all[0] = h1,
            //    h_all[r] = M_r h_all[r-1] + U_r
            ComposeArgs c;
            memset(&c, 0, sizeof(c));
            c.M = M;
            c.U = U;
            c.h0 = h1;
            c.h_in = hin;
            c.h_final = hin + (size_t)(R - 2) * N * p->H * K * V;
            c.R = R - 2;
            c.N = N;
            c.H = p->H;
            GDN_TRY(launched(launch_compose(K, V, c, s), who));
        }
        // 3. segments 1 .. R-1 emitted from those states; the last writes h_out
        ScanArgs e = a;
        e.ct = r.ct;
        e.ct.n_seg = R - 1;
        for (int i = 0; i < R; ++i) e.ct.seg_start[i] = r.ct.seg_start[i + 1];
        e.h_in = R == 2 ? h1 : hin;
        e.o = o;
        e.h_out = h_out;
        e.n_chains = N * (R - 1);
        return launched(launch_scan(K, V, C, dt, false, e, s), who);
    }
    // packed, some sequence cut into pieces: first pieces emitted and middle
    // pieces carried; the pieces' incoming states per sequence; the other
    // pieces emitted.  hs holds the state after each first piece (the final
    // state of a one-piece sequence), then every final state.
    float *hs = h_out ? h_out : h1;
    int ne, nc;
    packed_items(r, GDN_SCAN_HEAD_EMIT_CARRY, ne, nc);
    ScanArgs hd = a;
    hd.ct = r.ct;
    hd.h_in = h0;
    hd.o = o;
    hd.h_out = hs;
    hd.M_out = M;
    hd.U_out = U;
    hd.n_chains = r.ct.n_items;
    GDN_TRY(launched(launch_scan_head(K, V, C, dt, hd, h0, o, hs, s), who));
    ComposeArgs c;
    memset(&c, 0, sizeof(c));
    c.M = M;
    c.U = U;
    c.h0 = hs;
    c.h_in = hin;
    c.h_final = nullptr;
    c.R = 0;
    c.N = r.N;
    c.H = p->H;
    c.packed = 1;
    c.first = 1;
    for (int n = 0; n <= r.N; ++n) c.seq_first[n] = r.seq_first[n];
    GDN_TRY(launched(launch_compose(K, V, c, s), who));
    packed_items(r, GDN_SCAN_TAIL_EMIT, ne, nc);
    ScanArgs t = a;
    t.ct = r.ct;
    t.h_in = hin;
    t.o = o;
    t.h_out = hs;
    t.n_chains = r.ct.n_items;
    if (t.n_chains == 0) return GDN_OK;
    return launched(launch_scan(K, V, C, dt, false, t, s), who);
}

// Checks shared by the forward entry points (everything but the workspace).
static gdn_status forward_check(const gdn_problem *p, Resolved &r, const void *q, const void *k, const void *v,
                                const float *g, const float *beta, const float *h0, void *o, float *h_out) {
    GDN_TRY(resolve(p, r));
    const bool any = r.T > 0;
    GDN_TRY(check_ptr(q, "q", any));
    GDN_TRY(check_ptr(k, "k", any));
    GDN_TRY(check_ptr(v, "v", any));
    GDN_TRY(check_ptr(g, "g", any));
    GDN_TRY(check_ptr(beta, "beta", any));
    GDN_TRY(check_ptr(h0, "h0", false));
    GDN_TRY(check_ptr(o, "o", any));
    GDN_TRY(check_ptr(h_out, "h_out", false));
    return GDN_OK;
}

size_t gdn_forward_workspace_bytes(const gdn_problem *p) {
    Resolved r;
    if (resolve(p, r) != GDN_OK) return 0;
    return forward_layout(p, r).total;
}

gdn_status gdn_forward(const gdn_problem *p, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, const float *h0, void *o, float *h_out, void *workspace,
                       size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    Resolved r;
    GDN_TRY(forward_check(p, r, q, k, v, g, beta, h0, o, h_out));
    const FwdLayout L = forward_layout(p, r);
    GDN_TRY(check_ptr(workspace, "workspace", L.total > 0));
    if (L.total > 0 && workspace_bytes < L.total)
        return fail(GDN_EWORKSPACE, "forward workspace %zu bytes < %zu needed", workspace_bytes, L.total);
    if (L.total > 0) {
        const size_t es = elem_size(p->dtype);
        const size_t nst = (size_t)r.N * p->H * p->K * p->V * sizeof(float);
        const size_t no = (size_t)r.T * p->H * p->V * es;
        if (overlaps(workspace, L.total, o, no) || overlaps(workspace, L.total, h_out, nst) ||
            overlaps(workspace, L.total, h0, nst))
            return fail(GDN_EINVAL, "the workspace overlaps o, h0 or h_out");
    }
    return forward_run(p, r, q, k, v, g, beta, h0, o, h_out, static_cast<char *>(workspace), (hipStream_t)stream,
                       "gdn_forward");
}

// ---- gdn_forward_noalloc: gdn_forward with a scratch array instead of a workspace -------
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): gdn_forward's workspace lives in this
// file-scope device array, one copy on every GPU the library runs on, held
// until the process ends.  In host code `scratch` names a host-side stand-in;
// the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address reaches the kernels.
// Every call on a GPU uses that GPU's array, so calls that overlap on one GPU
// (other streams, other threads) race.  Nothing in it needs to start at zero:
// every byte a call reads there is written earlier in the same call.
static __device__ __align__(256) unsigned char scratch[GDN_FORWARD_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The scratch array's device address on the device of `stream` (the current
// device for the null stream).
gdn_status scratch_address(hipStream_t stream, char **out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(GDN_ELAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    dev = cur;
    if (stream) {
        e = hipStreamGetDevice(stream, &dev);
        if (e != hipSuccess) return fail(GDN_ELAUNCH, "hipStreamGetDevice: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(GDN_EUNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(GDN_ELAUNCH, "hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess || !ptr)
            return fail(GDN_ELAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return GDN_OK;
}
}  // namespace

gdn_status gdn_forward_noalloc(const gdn_problem *p, const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *h0, void *o, float *h_out, void *stream) {
    g_err[0] = 0;
    Resolved r;
    GDN_TRY(forward_check(p, r, q, k, v, g, beta, h0, o, h_out));
    const size_t need = forward_layout(p, r).total;
    if (need > GDN_FORWARD_SCRATCH_BYTES)
        return fail(GDN_EWORKSPACE, "the problem needs %zu bytes of scratch, more than the %zu bytes of "
                                    "gdn_forward_noalloc (use gdn_forward with a workspace)",
                    need, (size_t)GDN_FORWARD_SCRATCH_BYTES);
    char *ws = nullptr;
    if (need > 0) GDN_TRY(scratch_address((hipStream_t)stream, &ws));
    return forward_run(p, r, q, k, v, g, beta, h0, o, h_out, ws, (hipStream_t)stream, "gdn_forward_noalloc");
}

gdn_status gdn_segment_compose(int32_t R, int32_t N, int32_t H, int32_t K, int32_t V,
                               const float *M, const float *U, const float *h0, float *h_in,
                               float *h_final, void *stream) {
    g_err[0] = 0;
    if (R < 1 || N < 0 || H < 1 || K < 1 || V < 1)
        return fail(GDN_EINVAL, "bad sizes R=%d N=%d H=%d K=%d V=%d", R, N, H, K, V);
    if (!((K == 32 && V == 32) || (K == 128 && V == 128)))
        return fail(GDN_EUNSUPPORTED, "(K,V)=(%d,%d) not built", K, V);
    if (N == 0) return GDN_OK;
    GDN_TRY(check_ptr(M, "M", true));
    GDN_TRY(check_ptr(U, "U", true));
    GDN_TRY(check_ptr(h0, "h0", false));
    GDN_TRY(check_ptr(h_in, "h_in", true));
    GDN_TRY(check_ptr(h_final, "h_final", false));
    const size_t nh = (size_t)N * H;
    const size_t sz_state = (size_t)K * V * sizeof(float);
    const size_t sz_hin = R * nh * sz_state;
    if (overlaps(h_in, sz_hin, M, R * nh * K * K * sizeof(float)) ||
        overlaps(h_in, sz_hin, U, R * nh * sz_state) || overlaps(h_in, sz_hin, h0, nh * sz_state) ||
        overlaps(h_final, nh * sz_state, h_in, sz_hin) ||
        overlaps(h_final, nh * sz_state, M, R * nh * K * K * sizeof(float)) ||
        overlaps(h_final, nh * sz_state, U, R * nh * sz_state))
        return fail(GDN_EINVAL, "h_in / h_final must not alias the inputs or each other");
    ComposeArgs a;
    memset(&a, 0, sizeof(a));
    a.M = M;
    a.U = U;
    a.h0 = h0;
    a.h_in = h_in;
    a.h_final = h_final;
    a.R = R;
    a.N = N;
    a.H = H;
    (void)hipGetLastError();
    return launched(launch_compose(K, V, a, (hipStream_t)stream), "gdn_segment_compose");
}

gdn_status gdn_piece_compose(const gdn_problem *p, int32_t first, const float *M, const float *U,
                             const float *h_seed, float *h_in, float *h_final, void *stream) {
    g_err[0] = 0;
    Resolved r;
    GDN_TRY(resolve(p, r));
    if (!r.ct.packed) return fail(GDN_EINVAL, "gdn_piece_compose needs a packed problem (use gdn_segment_compose)");
    if (first != 0 && first != 1) return fail(GDN_EINVAL, "first = %d, must be 0 or 1", first);
    if (r.N == 0) return GDN_OK;
    // which buffers some sequence touches
    bool writes_in = false, reads_mu = false;
    for (int n = 0; n < r.N; ++n) {
        const int steps = r.seq_first[n + 1] - r.seq_first[n] - first;
        writes_in |= steps >= 1;
        reads_mu |= steps >= (h_final ? 1 : 2);
    }
    if (!writes_in && !h_final) return GDN_OK;   // nothing to do
    GDN_TRY(check_ptr(M, "M", reads_mu));
    GDN_TRY(check_ptr(U, "U", reads_mu));
    GDN_TRY(check_ptr(h_seed, "h_seed", false));
    GDN_TRY(check_ptr(h_in, "h_in", writes_in));
    GDN_TRY(check_ptr(h_final, "h_final", false));
    const size_t state = (size_t)p->H * p->K * p->V * sizeof(float);
    const size_t sz_in = r.P * state, sz_seq = r.N * state, sz_m = (size_t)r.P * p->H * p->K * p->K * sizeof(float);
    if (overlaps(h_in, sz_in, M, sz_m) || overlaps(h_in, sz_in, U, sz_in) || overlaps(h_in, sz_in, h_seed, sz_seq) ||
        overlaps(h_final, sz_seq, h_in, sz_in) || overlaps(h_final, sz_seq, M, sz_m) ||
        overlaps(h_final, sz_seq, U, sz_in))
        return fail(GDN_EINVAL, "h_in / h_final must not alias the inputs or each other");
    ComposeArgs a;
    memset(&a, 0, sizeof(a));
    a.M = M;
    a.U = U;
    a.h0 = h_seed;
    a.h_in = h_in;
    a.h_final = h_final;
    a.R = 0;
    a.N = r.N;
    a.H = p->H;
    a.packed = 1;
    a.first = first;
    for (int n = 0; n <= r.N; ++n) a.seq_first[n] = r.seq_first[n];
    (void)hipGetLastError();
    return launched(launch_compose(p->K, p->V, a, (hipStream_t)stream), "gdn_piece_compose");
}

gdn_status gdn_decode_step(int32_t B, int32_t H, int32_t H_qk, int32_t K, int32_t V, int32_t dtype,
                           const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, void *o, void *stream) {
    g_err[0] = 0;
    if (B < 0 || H < 1 || K < 1 || V < 1)
        return fail(GDN_EINVAL, "bad sizes B=%d H=%d K=%d V=%d", B, H, K, V);
    if (H_qk < 1 || H_qk > H || H % H_qk != 0)
        return fail(GDN_EINVAL, "H_qk = %d must divide H = %d", H_qk, H);
    if (!((K == 32 && V == 32) || (K == 128 && V == 128)))
        return fail(GDN_EUNSUPPORTED, "(K,V)=(%d,%d) not built", K, V);
    if (dtype != GDN_F32 && dtype != GDN_BF16)
        return fail(GDN_EUNSUPPORTED, "dtype %d not supported", dtype);
    if (B == 0) return GDN_OK;
    if ((int64_t)B * H > 0x7fffffffLL) return fail(GDN_EUNSUPPORTED, "B*H too large");
    GDN_TRY(check_ptr(q, "q", true));
    GDN_TRY(check_ptr(k, "k", true));
    GDN_TRY(check_ptr(v, "v", true));
    GDN_TRY(check_ptr(g, "g", true));
    GDN_TRY(check_ptr(beta, "beta", true));
    GDN_TRY(check_ptr(state, "state", true));
    GDN_TRY(check_ptr(o, "o", true));
    DecodeArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.o = o;
    a.B = B;
    a.H = H;
    a.Hk = H_qk;
    (void)hipGetLastError();
    return launched(launch_decode(K, V, dtype, a, (hipStream_t)stream), "gdn_decode_step");
}

gdn_status gdn_causal_conv1d(int32_t B, int32_t S, int32_t D, int32_t W, int32_t dtype, int32_t activation,
                             const int32_t *cu_seqlens, int32_t n_seqs, const void *x, const void *weight,
                             const void *state_in, void *state_out, void *y, void *stream) {
    g_err[0] = 0;
    if (B < 0 || S < 0 || D < 1 || W < 1 || W > 8)
        return fail(GDN_EINVAL, "bad sizes B=%d S=%d D=%d W=%d (1 <= W <= 8)", B, S, D, W);
    if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_EUNSUPPORTED, "dtype %d not supported", dtype);
    if (activation != 0 && activation != 1) return fail(GDN_EINVAL, "activation %d (0 or 1)", activation);
    if ((int64_t)D > 65535LL * 256) return fail(GDN_EUNSUPPORTED, "D = %d too large", D);
    ConvArgs a;
    memset(&a, 0, sizeof(a));
    if (cu_seqlens) {
        if (B != 1) return fail(GDN_EINVAL, "packed mode needs B == 1 (got %d)", B);
        if (n_seqs < 1 || n_seqs > GDN_MAX_SEQS) return fail(GDN_EINVAL, "n_seqs %d not in 1 .. GDN_MAX_SEQS", n_seqs);
        if (cu_seqlens[0] != 0) return fail(GDN_EORDER, "cu_seqlens[0] = %d, must be 0", cu_seqlens[0]);
        for (int n = 0; n < n_seqs; ++n)
            if (cu_seqlens[n + 1] < cu_seqlens[n])
                return fail(GDN_EORDER, "cu_seqlens decreases at %d (%d -> %d)", n, cu_seqlens[n], cu_seqlens[n + 1]);
        if (cu_seqlens[n_seqs] != S) return fail(GDN_EINVAL, "cu_seqlens[n_seqs] = %d != S = %d", cu_seqlens[n_seqs], S);
        for (int n = 0; n <= n_seqs; ++n) a.start[n] = cu_seqlens[n];
        a.packed = 1;
        a.N = n_seqs;
        a.T = S;
    } else {
        if ((int64_t)B > GDN_MAX_SEQS * 1024LL) return fail(GDN_EUNSUPPORTED, "B = %d too large", B);
        a.N = B;
        a.T = (int64_t)B * S;
    }
    const int N = a.N;
    if (N == 0) return GDN_OK;
    const bool any = a.T > 0;
    GDN_TRY(check_ptr(x, "x", any));
    GDN_TRY(check_ptr(y, "y", any));
    GDN_TRY(check_ptr(weight, "weight", any || state_out));
    GDN_TRY(check_ptr(state_in, "state_in", false));
    GDN_TRY(check_ptr(state_out, "state_out", false));
    const size_t es = dtype == GDN_F32 ? 4 : 2;
    const size_t xbytes = (size_t)a.T * D * es, sbytes = (size_t)N * D * (W - 1) * es;
    if (overlaps(x, xbytes, y, xbytes)) return fail(GDN_EINVAL, "y must not overlap x");
    if (state_out && state_in && overlaps(state_in, sbytes, state_out, sbytes)) {
        // a sequence spread over two token blocks (of 8 tokens or more, laid out
        // per sequence or along the token axis in blocks of 64) would read its
        // state in one block while another block writes it
        for (int n = 0; n < N; ++n) {
            const int64_t s0 = a.packed ? a.start[n] : (int64_t)n * S, s1 = a.packed ? a.start[n + 1] : s0 + S;
            if (s1 - s0 > 8 || (s1 > s0 && s0 / 64 != (s1 - 1) / 64))
                return fail(GDN_EINVAL, "state_out may alias state_in only when every sequence has at most 8 tokens "
                                        "within one multiple of 64 (sequence %d spans %lld .. %lld)",
                            n, (long long)s0, (long long)s1);
        }
    }
    a.x = x;
    a.weight = weight;
    a.state_in = state_in;
    a.state_out = state_out;
    a.y = y;
    a.D = D;
    a.W = W;
    a.S = S;
    a.activation = activation;
    if (!any && !state_out) return GDN_OK;
    (void)hipGetLastError();
    return launched(launch_causal_conv(dtype, a, (hipStream_t)stream), "gdn_causal_conv1d");
}

gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t V, int32_t dtype, float eps, const void *o, const void *z,
                             const float *weight, void *y, void *stream) {
    g_err[0] = 0;
    if (rows < 0 || V < 1 || V > 256) return fail(GDN_EINVAL, "bad sizes rows=%lld V=%d (1 <= V <= 256)",
                                                  (long long)rows, V);
    if (!(eps >= 0.f)) return fail(GDN_EINVAL, "eps must be >= 0");
    if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_EUNSUPPORTED, "dtype %d not supported", dtype);
    if (rows == 0) return GDN_OK;
    GDN_TRY(check_ptr(o, "o", true));
    GDN_TRY(check_ptr(z, "z", false));
    GDN_TRY(check_ptr(weight, "weight", true));
    GDN_TRY(check_ptr(y, "y", true));
    const size_t bytes = (size_t)rows * V * (dtype == GDN_F32 ? 4 : 2);
    if (y != o && overlaps(o, bytes, y, bytes)) return fail(GDN_EINVAL, "y must be o or not overlap it");
    if (z && overlaps(z, bytes, y, bytes)) return fail(GDN_EINVAL, "y must not overlap z");
    NormArgs a;
    a.o = o;
    a.z = z;
    a.weight = weight;
    a.y = y;
    a.rows = rows;
    a.V = V;
    a.eps = eps;
    (void)hipGetLastError();
    return launched(launch_gated_rmsnorm(dtype, a, (hipStream_t)stream), "gdn_gated_rmsnorm");
}

// Workspace of the backward pass, per (chunk, head), fp32: T, attn, Ak
// (C x C), w (C x K), u, delta, ddelta (C x V), state, dstate (K x V).
static size_t backward_ws_per_chunk(const gdn_problem *p) {
    return sizeof(float) * ((size_t)3 * p->C * p->C + (size_t)p->C * p->K + (size_t)3 * p->C * p->V +
                            (size_t)2 * p->K * p->V);
}

// The backward pass runs the chains of the forward's schedule: a sequence cut
// into segments (batch) or pieces (packed) scans each part in parallel, from
// boundary states composed of the parts' carries.
static gdn_status backward_problem(const gdn_problem *p, Resolved &r) { return resolve(p, r); }

static bool grouped(const gdn_problem *p) { return p->H_qk != 0 && p->H_qk != p->H; }

// chains that split sequences need carries and boundary states
static bool split_chains(const Resolved &r) { return r.P > r.N; }

// per-chunk-head workspace; then (grouped key heads) dq, dk of every value
// head; then (split chains), per chain and head, M and Mt [K,K] and U, E,
// h_in, dh_in [K,V] (fp32)
static size_t backward_ws_bytes(const gdn_problem *p, const Resolved &r) {
    size_t n = (size_t)r.n_chunks * p->H * backward_ws_per_chunk(p);
    if (grouped(p)) n += 2 * (size_t)r.T * p->H * p->K * sizeof(float);
    if (split_chains(r))
        n += (size_t)r.P * p->H * sizeof(float) * ((size_t)2 * p->K * p->K + (size_t)4 * p->K * p->V);
    return n;
}

size_t gdn_backward_workspace_bytes(const gdn_problem *p) {
    Resolved r;
    if (backward_problem(p, r) != GDN_OK) return 0;
    return backward_ws_bytes(p, r);
}

gdn_status gdn_backward(const gdn_problem *p, const void *q, const void *k, const void *v,
                        const float *g, const float *beta, const float *h0, const void *dout,
                        const float *dhT, void *dq, void *dk, void *dv, float *dg, float *dbeta,
                        float *dh0, void *workspace, size_t workspace_bytes, void *stream) {
    g_err[0] = 0;
    Resolved r;
    GDN_TRY(backward_problem(p, r));
    const bool any = r.T > 0;
    GDN_TRY(check_ptr(q, "q", any));
    GDN_TRY(check_ptr(k, "k", any));
    GDN_TRY(check_ptr(v, "v", any));
    GDN_TRY(check_ptr(g, "g", any));
    GDN_TRY(check_ptr(beta, "beta", any));
    GDN_TRY(check_ptr(h0, "h0", false));
    GDN_TRY(check_ptr(dout, "dout", any));
    GDN_TRY(check_ptr(dhT, "dhT", false));
    GDN_TRY(check_ptr(dq, "dq", any));
    GDN_TRY(check_ptr(dk, "dk", any));
    GDN_TRY(check_ptr(dv, "dv", any));
    GDN_TRY(check_ptr(dg, "dg", any));
    GDN_TRY(check_ptr(dbeta, "dbeta", any));
    GDN_TRY(check_ptr(dh0, "dh0", false));
    const size_t need = backward_ws_bytes(p, r);
    GDN_TRY(check_ptr(workspace, "workspace", need > 0));
    if (workspace_bytes < need)
        return fail(GDN_EWORKSPACE, "backward workspace %zu bytes < %zu needed", workspace_bytes, need);
    const size_t es = elem_size(p->dtype);
    const int Hk = p->H_qk > 0 ? p->H_qk : p->H;
    const size_t nqk = (size_t)r.T * Hk * p->K * es, nv = (size_t)r.T * p->H * p->V * es;
    const size_t ngb = (size_t)r.T * p->H * sizeof(float);
    const size_t nst = (size_t)r.N * p->H * p->K * p->V * sizeof(float);
    const struct { const void *ptr; size_t n; } ins[] = {
        {q, nqk}, {k, nqk}, {v, nv}, {g, ngb}, {beta, ngb}, {h0, nst}, {dout, nv}, {dhT, nst},
        {workspace, need}};
    const struct { const void *ptr; size_t n; const char *name; } outs[] = {
        {dq, nqk, "dq"}, {dk, nqk, "dk"}, {dv, nv, "dv"}, {dg, ngb, "dg"}, {dbeta, ngb, "dbeta"},
        {dh0, nst, "dh0"}};
    for (const auto &o : outs) {
        for (const auto &in : ins)
            if (overlaps(o.ptr, o.n, in.ptr, in.n))
                return fail(GDN_EINVAL, "%s overlaps an input or the workspace", o.name);
        for (const auto &o2 : outs)
            if (&o2 != &o && overlaps(o.ptr, o.n, o2.ptr, o2.n))
                return fail(GDN_EINVAL, "%s overlaps another output", o.name);
    }
    if (!any && !dh0) return GDN_OK;
    // (with no tokens only the reverse scan runs: it writes dh0 = dhT, or 0)
    BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.dout = dout;
    a.g = g;
    a.beta = beta;
    a.h0 = h0;
    a.dhT = dhT;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dg = dg;
    a.dbeta = dbeta;
    a.dh0 = dh0;
    const size_t CH = (size_t)r.n_chunks * p->H;
    float *ws = static_cast<float *>(workspace);
    const size_t CC = (size_t)p->C * p->C;
    a.T = ws;
    a.attn = a.T + CH * CC;
    a.Ak = a.attn + CH * CC;
    a.w = a.Ak + CH * CC;
    a.u = a.w + CH * p->C * p->K;
    a.d = a.u + CH * p->C * p->V;
    a.dd = a.d + CH * p->C * p->V;
    a.hs = a.dd + CH * p->C * p->V;
    a.dhs = a.hs + CH * p->K * p->V;
    a.dq_acc = a.dk_acc = nullptr;
    float *tail = a.dhs + CH * p->K * p->V;
    if (grouped(p)) {
        a.dq_acc = tail;
        a.dk_acc = a.dq_acc + (size_t)r.T * p->H * p->K;
        tail = a.dk_acc + (size_t)r.T * p->H * p->K;
    }
    a.h_in = a.dh_in = nullptr;
    a.M = a.Mt = a.U = a.E = nullptr;
    ComposeArgs fwd, rev;
    const bool split = split_chains(r);
    if (split) {
        const size_t KK = (size_t)r.P * p->H * p->K * p->K, KV = (size_t)r.P * p->H * p->K * p->V;
        a.M = tail;
        a.Mt = a.M + KK;
        a.U = a.Mt + KK;
        a.E = a.U + KV;
        float *hin = a.E + KV, *dhin = hin + KV;
        a.h_in = hin;
        a.dh_in = dhin;
        memset(&fwd, 0, sizeof(fwd));
        fwd.R = r.R;
        fwd.N = r.N;
        fwd.H = p->H;
        fwd.packed = r.ct.packed;
        fwd.first = 0;
        for (int n = 0; n <= r.N && r.ct.packed; ++n) fwd.seq_first[n] = r.seq_first[n];
        rev = fwd;
        fwd.M = a.M;        // h_in[next] = M h_in + U, from h0
        fwd.U = a.U;
        fwd.h0 = h0;
        fwd.h_in = hin;
        rev.M = a.Mt;       // dh_in[previous] = Mt dh_in + E, from dhT
        rev.U = a.E;
        rev.h0 = dhT;
        rev.h_in = dhin;
        rev.reverse = 1;
    }
    a.carry = 0;
    a.N = r.N;
    a.H = p->H;
    a.Hk = Hk;
    a.tokens = r.T;
    a.n_chunks = r.n_chunks;
    a.ct = r.ct;
    (void)hipGetLastError();
    return launched(launch_backward(p->K, p->V, p->C, p->dtype, a, r.P, split ? &fwd : nullptr,
                                    split ? &rev : nullptr, (hipStream_t)stream),
                    "gdn_backward");
}

int32_t gdn_scan_backend(const gdn_problem *p) {
    Resolved r;
    if (resolve(p, r) != GDN_OK) return -1;
    return mfma_scan_available(p->K, p->V, p->C, p->dtype) ? 1 : 0;
}

const char *gdn_status_string(int32_t status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_EINVAL: return "GDN_EINVAL: invalid argument";
        case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED: shape or dtype not supported";
        case GDN_EORDER: return "GDN_EORDER: segments or sequences not contiguous and in order";
        case GDN_ELAUNCH: return "GDN_ELAUNCH: kernel launch failed";
        case GDN_EWORKSPACE: return "GDN_EWORKSPACE: workspace smaller than the problem needs";
        default: return "unknown gdn_status";
    }
}

const char *gdn_last_error(void) { return g_err; }

int32_t gdn_version(void) { return 120; }

}  // extern "C"
