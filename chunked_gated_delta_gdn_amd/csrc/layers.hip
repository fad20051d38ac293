// The steps on either side of the core: the depthwise causal convolution over
// the q, k, v channels before it (MaxText PR "Add context parallelism to the
// Gated Delta Net", section "Implementation": a causal conv1d whose halo is
// kernel_dim - 1 tokens; "RFC(qwen35): TP Phase 2", section "Partition
// Contract": a conv state of qkv_dim x (kernel_dim - 1) per request) and the
// gated RMSNorm after it (same RFC, section "Execution Contract").
//
//   conv:  y[t, c] = act(sum_i w[c, i] x[t - (W-1) + i, c]), positions before a
//          sequence's start taken from its state (W-1 tokens, oldest first),
//          the state afterwards being the last W-1 positions; act = identity
//          or SiLU.
//   norm:  y = o / sqrt(mean(o^2) + eps) * weight * SiLU(z), per row of V.
//
// Both stream HBM once (read x, write y; read o, z, write y), so they are laid
// out for coalescing: consecutive lanes take consecutive channels (conv) or
// consecutive elements of a row (norm), and every value is read once.
#include "dev_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kConvThreads = 256;   // channels per workgroup
constexpr int kConvTokens = 64;     // tokens per thread (one token block)
constexpr int kMaxTaps = 8;

// u sigmoid(u), with the hardware reciprocal (about 1 ulp) in place of a full
// division: large negative u gives 1 + exp(-u) = inf and a zero result, as
// the quotient does.
__device__ __forceinline__ float silu(float u) { return u * __builtin_amdgcn_rcpf(1.f + __expf(-u)); }

// Sequence n of token t (packed: last n with start[n] <= t; batch: t / S).
__device__ __forceinline__ int seq_of(const ConvArgs &a, int64_t t) {
    if (!a.packed) return (int)(t / a.S);
    int lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.start[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}
__device__ __forceinline__ int64_t seq_start(const ConvArgs &a, int n) {
    return a.packed ? (int64_t)a.start[n] : (int64_t)n * a.S;
}
__device__ __forceinline__ int64_t seq_end(const ConvArgs &a, int n) {
    return a.packed ? (int64_t)a.start[n + 1] : (int64_t)(n + 1) * a.S;
}

template <typename T>
__global__ __launch_bounds__(kConvThreads) void causal_conv_kernel(ConvArgs a) {
    const int64_t c = (int64_t)blockIdx.y * kConvThreads + threadIdx.x;
    if (c >= a.D) return;
    const int W = a.W, P = W - 1;
    const int64_t D = a.D;
    float w[kMaxTaps];
#pragma unroll
    for (int i = 0; i < kMaxTaps; ++i) w[i] = i < W ? Elem<T>::load(a.weight, c * W + i) : 0.f;
    if ((int64_t)blockIdx.x * kConvTokens >= a.T) {
        // the extra block column: sequences with no tokens keep their state
        if (!a.state_out) return;
        for (int n = 0; n < a.N; ++n) {
            if (seq_end(a, n) != seq_start(a, n)) continue;
            for (int i = 0; i < P; ++i)
                Elem<T>::store(a.state_out, ((int64_t)n * D + c) * P + i,
                               a.state_in ? Elem<T>::load(a.state_in, ((int64_t)n * D + c) * P + i) : 0.f);
        }
        return;
    }
    const int64_t t0 = (int64_t)blockIdx.x * kConvTokens;
    const int64_t t1 = t0 + kConvTokens < a.T ? t0 + kConvTokens : a.T;
    int n = seq_of(a, t0);
    int64_t s0 = seq_start(a, n), s1 = seq_end(a, n);
    // the window: win[P-1-j] = x~[t - 1 - j] for the token t about to be processed
    float win[kMaxTaps];
    auto prev = [&](int64_t tau) -> float {   // x~ at position tau of sequence n (tau < t)
        if (tau >= s0) return Elem<T>::load(a.x, tau * D + c);
        const int64_t back = s0 - tau;        // 1 .. P
        return a.state_in ? Elem<T>::load(a.state_in, ((int64_t)n * D + c) * P + (P - back)) : 0.f;
    };
#pragma unroll
    for (int j = 0; j < kMaxTaps; ++j)
        if (j < P) win[j] = prev(t0 - P + j);
    for (int64_t t = t0; t < t1; ++t) {
        if (t == s1) {
            // next sequence: its window starts from its own state
            do {
                ++n;
                s0 = seq_start(a, n);
                s1 = seq_end(a, n);
            } while (s1 == s0);   // (empty sequences; t < T, so a sequence holds t)
#pragma unroll
            for (int j = 0; j < kMaxTaps; ++j)
                if (j < P) win[j] = a.state_in ? Elem<T>::load(a.state_in, ((int64_t)n * D + c) * P + j) : 0.f;
        }
        const float xt = Elem<T>::load(a.x, t * D + c);
        float acc = w[P] * xt;
#pragma unroll
        for (int j = 0; j < kMaxTaps; ++j)
            if (j < P) acc = fmaf(w[j], win[j], acc);
        Elem<T>::store(a.y, t * D + c, a.activation ? silu(acc) : acc);
#pragma unroll
        for (int j = 0; j + 1 < kMaxTaps; ++j)
            if (j + 1 < P) win[j] = win[j + 1];
        if (P > 0) win[P - 1] = xt;
        if (t == s1 - 1 && a.state_out) {
#pragma unroll
            for (int j = 0; j < kMaxTaps; ++j)
                if (j < P) Elem<T>::store(a.state_out, ((int64_t)n * D + c) * P + j, win[j]);
        }
    }
}

// One wave per row of V elements; lane l takes elements l, l + 64, ...
template <typename T>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * 256) >> 6;
    const int V = a.V;
    constexpr int kMaxPer = 4;   // V <= 256
    for (int64_t r = wave; r < a.rows; r += n_waves) {
        float o[kMaxPer];
        float ss = 0.f;
#pragma unroll
        for (int m = 0; m < kMaxPer; ++m) {
            const int i = lane + 64 * m;
            o[m] = i < V ? Elem<T>::load(a.o, r * V + i) : 0.f;
            ss = fmaf(o[m], o[m], ss);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = rsqrtf(ss / (float)V + a.eps);
#pragma unroll
        for (int m = 0; m < kMaxPer; ++m) {
            const int i = lane + 64 * m;
            if (i >= V) continue;
            float yv = o[m] * inv * a.weight[i];
            if (a.z) yv *= silu(Elem<T>::load(a.z, r * V + i));
            Elem<T>::store(a.y, r * V + i, yv);
        }
    }
}

// 8 consecutive channels per thread as one 16-byte (bf16) or 32-byte (fp32)
// access per token, for D a multiple of 8: a wave moves 512 channels of a token
// per load instead of 64.
template <typename T> struct Vec8;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
template <> struct Vec8<bf16_t> {
    static __device__ __forceinline__ void unpack(const u32x4v &u, float (&v)[8]) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(u[k] << 16);
            v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ u32x4v pack(const float (&v)[8]) {
        // two values per v_cvt_pk_bf16_f32 (round to nearest even)
        u32x4v w;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){v[2 * k], v[2 * k + 1]}, bf16x2));
        return w;
    }
    static __device__ __forceinline__ void load(const void *p, int64_t i, float (&v)[8]) {
        unpack(*reinterpret_cast<const u32x4v *>(static_cast<const uint16_t *>(p) + i), v);
    }
    static __device__ __forceinline__ void store(void *p, int64_t i, const float (&v)[8]) {
        *reinterpret_cast<u32x4v *>(static_cast<uint16_t *>(p) + i) = pack(v);
    }
    // streaming (non-temporal) access for data read or written once
    static __device__ __forceinline__ void load_nt(const void *p, int64_t i, float (&v)[8]) {
        unpack(__builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(static_cast<const uint16_t *>(p) + i)), v);
    }
    static __device__ __forceinline__ void store_nt(void *p, int64_t i, const float (&v)[8]) {
        __builtin_nontemporal_store(pack(v), reinterpret_cast<u32x4v *>(static_cast<uint16_t *>(p) + i));
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const void *p, int64_t i, float (&v)[8]) {
        const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
        const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store(void *p, int64_t i, const float (&v)[8]) {
        float *q = static_cast<float *>(p) + i;
        *reinterpret_cast<float4 *>(q) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4 *>(q + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
    static __device__ __forceinline__ void load_nt(const void *p, int64_t i, float (&v)[8]) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        const f4v a = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(static_cast<const float *>(p) + i));
        const f4v b = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(static_cast<const float *>(p) + i + 4));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = a[k];
            v[4 + k] = b[k];
        }
    }
    static __device__ __forceinline__ void store_nt(void *p, int64_t i, const float (&v)[8]) {
        typedef float f4v __attribute__((ext_vector_type(4)));
        float *q = static_cast<float *>(p) + i;
        __builtin_nontemporal_store((f4v){v[0], v[1], v[2], v[3]}, reinterpret_cast<f4v *>(q));
        __builtin_nontemporal_store((f4v){v[4], v[5], v[6], v[7]}, reinterpret_cast<f4v *>(q + 4));
    }
};

// One token's 8 channels as loaded (packed: a uint4 of 8 bf16, or two float4),
// unpacked to fp32 where used.  Plain vector arrays, which the compiler keeps in
// registers (arrays of structs of this size went to scratch memory).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Raw8 { typedef u32x4 type; static constexpr int n = 1; };
template <> struct Raw8<float> { typedef float4 type; static constexpr int n = 2; };
__device__ __forceinline__ void raw_load(u32x4 (&r)[1], const void *p, int64_t i) {
    r[0] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p) + i);
}
__device__ __forceinline__ void raw_load(float4 (&r)[2], const void *p, int64_t i) {
    r[0] = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i);
    r[1] = *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + i + 4);
}
__device__ __forceinline__ void raw_unpack(const u32x4 (&r)[1], float (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(r[0][k] << 16);
        v[2 * k + 1] = __uint_as_float(r[0][k] & 0xffff0000u);
    }
}
__device__ __forceinline__ void raw_unpack(const float4 (&r)[2], float (&v)[8]) {
    v[0] = r[0].x; v[1] = r[0].y; v[2] = r[0].z; v[3] = r[0].w;
    v[4] = r[1].x; v[5] = r[1].y; v[6] = r[1].z; v[7] = r[1].w;
}

// The same convolution, 8 channels per thread (D % 8 == 0), streaming a run of
// kConvRun tokens: the run is read in stages of TS tokens (one 16-byte bf16 or
// 32-byte fp32 access per token), the loads of the next stage are issued
// before the current one is computed, and the W-1 window of past tokens stays
// in registers from one stage to the next, so only a run's first token reads
// a halo (from its sequence's state or the tokens before the run).  Runs are
// laid out per sequence (block_start[n] .. block_start[n+1]-1 hold sequence
// n), so a run never crosses a sequence boundary.  (Measured on the
// 65,536-token x 8,192-channel bf16 case against 8-token blocks whose threads
// issue all loads, compute and exit.)
template <typename T> constexpr int conv_stage() { return sizeof(T) == 2 ? 8 : 4; }
// Workgroup b works on channel group b % G and run b / G (G = gridDim of the
// channel groups, passed as n_cg): the channel groups of one run are
// dispatched together, so the reads and writes of a run's token rows arrive
// as whole rows.
constexpr int kConvRun = 64;

template <typename T, int MT>   // MT: at least W (4 or 8), the size of the tap and window arrays
__global__ __launch_bounds__(kConvThreads) void causal_conv_run_kernel(ConvArgs a) {
    constexpr int TS = conv_stage<T>();
    constexpr int NR = Raw8<T>::n;
    typedef typename Raw8<T>::type raw_t;
    const uint32_t bid = blockIdx.x, ncg = (uint32_t)a.n_cg;   // (wave uniform)
    const int64_t cg = bid % ncg, bx = bid / ncg;
    const int64_t c = (cg * kConvThreads + threadIdx.x) * 8;   // first channel
    if (c >= a.D) return;
    const int W = a.W, P = W - 1;
    const int64_t D = a.D;
    auto state_at = [&](int n, int k, int j) -> float {   // state of channel c + k, position j (oldest first)
        return a.state_in ? Elem<T>::load(a.state_in, ((int64_t)n * D + c + k) * P + j) : 0.f;
    };
    if (bx >= a.n_blocks) {
        // the extra block column: sequences with no tokens keep their state
        if (!a.state_out) return;
        for (int n = 0; n < a.N; ++n) {
            if (seq_end(a, n) != seq_start(a, n)) continue;
            for (int k = 0; k < 8; ++k)
                for (int j = 0; j < P; ++j) Elem<T>::store(a.state_out, ((int64_t)n * D + c + k) * P + j, state_at(n, k, j));
        }
        return;
    }
    int n;
    int64_t r_in_seq;
    if (a.packed) {
        int lo = 0, hi = a.N - 1;   // last n with block_start[n] <= bx
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.block_start[mid] <= bx) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        r_in_seq = bx - a.block_start[n];
    } else {
        const int64_t rps = (a.S + kConvRun - 1) / kConvRun;
        n = (int)(bx / rps);
        r_in_seq = bx % rps;
    }
    const int64_t s0 = seq_start(a, n), s1 = seq_end(a, n);
    const int64_t t0 = s0 + r_in_seq * kConvRun;
    const int nt = (int)(s1 - t0 < kConvRun ? s1 - t0 : kConvRun);
    const int nst = (nt + TS - 1) / TS;
    raw_t xa[TS][NR], xb[TS][NR];
    // (tokens past the run's end re-read its last token: every load is
    // unconditional, and their values are not used)
#define GDN_CONV_LOAD_STAGE(xs, st)                                         \
    _Pragma("unroll") for (int u = 0; u < TS; ++u) {                        \
        const int tok = (st) * TS + u < nt ? (st) * TS + u : nt - 1;       \
        raw_load(xs[u], a.x, (t0 + tok) * D + c);                           \
    }
    GDN_CONV_LOAD_STAGE(xa, 0)
    float w[8][MT];
    if (MT == 4 && W == 4) {
        // the 8 channels' 32 taps are contiguous: 4 accesses of 8 values
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float t8[8];
            Vec8<T>::load(a.weight, c * 4 + 8 * q, t8);
#pragma unroll
            for (int e = 0; e < 8; ++e) w[2 * q + e / 4][e % 4] = t8[e];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int i = 0; i < MT; ++i) w[k][i] = i < W ? Elem<T>::load(a.weight, (c + k) * W + i) : 0.f;
    }
    // the tap on the current token, picked without a run-time array index (which
    // would put w in scratch memory)
    float wl[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        wl[k] = 0.f;
#pragma unroll
        for (int i = 0; i < MT; ++i)
            if (i == P) wl[k] = w[k][i];
    }
    float win[MT][8];   // win[j] = x~[t - P + j] for the token t about to be processed
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        if (j >= P) continue;
        const int64_t tau = t0 - P + j;
        if (tau >= s0) {
            Vec8<T>::load(a.x, tau * D + c, win[j]);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) win[j][k] = state_at(n, k, (int)(P - (s0 - tau)));
        }
    }
#define GDN_CONV_RUN_STAGE(xs, st)                                                          \
    _Pragma("unroll") for (int u = 0; u < TS; ++u) {                                        \
        if ((st) * TS + u < nt) {                                                           \
            float xv[8], out[8];                                                            \
            raw_unpack(xs[u], xv);                                                          \
            _Pragma("unroll") for (int k = 0; k < 8; ++k) {                                 \
                float acc = wl[k] * xv[k];                                                  \
                _Pragma("unroll") for (int j = 0; j < MT; ++j)                              \
                    if (j < P) acc = fmaf(w[k][j], win[j][k], acc);                         \
                out[k] = a.activation ? silu(acc) : acc;                                    \
            }                                                                               \
            Vec8<T>::store(a.y, (t0 + (st) * TS + u) * D + c, out);                         \
            _Pragma("unroll") for (int j = 0; j + 1 < MT; ++j)                              \
                if (j + 1 < P)                                                              \
                    _Pragma("unroll") for (int k = 0; k < 8; ++k) win[j][k] = win[j + 1][k]; \
            _Pragma("unroll") for (int j = 0; j < MT; ++j)                                  \
                if (j == P - 1)                                                             \
                    _Pragma("unroll") for (int k = 0; k < 8; ++k) win[j][k] = xv[k];        \
        }                                                                                   \
    }
    // two register sets with fixed homes: stage st in xa (st even) or xb (odd)
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst) { GDN_CONV_LOAD_STAGE(xb, st + 1) }
        GDN_CONV_RUN_STAGE(xa, st)
        if (st + 1 >= nst) break;
        if (st + 2 < nst) { GDN_CONV_LOAD_STAGE(xa, st + 2) }
        GDN_CONV_RUN_STAGE(xb, st + 1)
    }
#undef GDN_CONV_LOAD_STAGE
#undef GDN_CONV_RUN_STAGE
    if (t0 + nt == s1 && a.state_out) {
        // the run holding the sequence's last token writes its state
#pragma unroll
        for (int j = 0; j < MT; ++j)
            if (j < P)
#pragma unroll
                for (int k = 0; k < 8; ++k) Elem<T>::store(a.state_out, ((int64_t)n * D + c + k) * P + j, win[j][k]);
    }
}

// bf16 with at most 4 taps: the same runs and stages, with the taps applied as
// bf16 dot products (v_dot2_f32_bf16, fp32 sums) on pairs of consecutive
// tokens.  Taps are padded at the front to four (w~_i = w_{i-(4-W)}, zero
// before), so y[t] = dot(w~_0, w~_1; x[t-3], x[t-2]) + dot(w~_2, w~_3; x[t-1],
// x[t]), and each token forms one pair (x[t-1], x[t]) per channel, used for
// its own output and for the output two tokens later.  Positions before a
// sequence's start come from its state (W-1 positions) and are zero beyond it
// (their taps are zero).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2bf(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w), __builtin_bit_cast(bf16x2v, x), acc, false);
}
// (x[t-1], x[t]) of the low / high channel of a 32-bit pair of channels
__device__ __forceinline__ uint32_t pair_lo(uint32_t prev, uint32_t cur) { return __builtin_amdgcn_perm(cur, prev, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t prev, uint32_t cur) { return __builtin_amdgcn_perm(cur, prev, 0x07060302u); }

__global__ __launch_bounds__(kConvThreads) void causal_conv_run_bf16w4_kernel(ConvArgs a) {
    constexpr int TS = 8;
    const uint32_t bid = blockIdx.x, ncg = (uint32_t)a.n_cg;   // (wave uniform)
    const int64_t cg = bid % ncg, bx = bid / ncg;
    const int64_t c = (cg * kConvThreads + threadIdx.x) * 8;   // first channel
    if (c >= a.D) return;
    const int W = a.W, P = W - 1;
    const int64_t D = a.D;
    const uint16_t *xs16 = static_cast<const uint16_t *>(a.x);
    const uint16_t *st16 = static_cast<const uint16_t *>(a.state_in);
    if (bx >= a.n_blocks) {
        // the extra block column: sequences with no tokens keep their state
        if (!a.state_out) return;
        uint16_t *so = static_cast<uint16_t *>(a.state_out);
        for (int n = 0; n < a.N; ++n) {
            if (seq_end(a, n) != seq_start(a, n)) continue;
            for (int k = 0; k < 8; ++k)
                for (int j = 0; j < P; ++j) {
                    const int64_t i = ((int64_t)n * D + c + k) * P + j;
                    so[i] = st16 ? st16[i] : 0;
                }
        }
        return;
    }
    int n;
    int64_t r_in_seq;
    if (a.packed) {
        int lo = 0, hi = a.N - 1;   // last n with block_start[n] <= bx
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.block_start[mid] <= bx) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        r_in_seq = bx - a.block_start[n];
    } else {
        const int64_t rps = (a.S + kConvRun - 1) / kConvRun;
        n = (int)(bx / rps);
        r_in_seq = bx % rps;
    }
    const int64_t s0 = seq_start(a, n), s1 = seq_end(a, n);
    const int64_t t0 = s0 + r_in_seq * kConvRun;
    const int nt = (int)(s1 - t0 < kConvRun ? s1 - t0 : kConvRun);
    const int nst = (nt + TS - 1) / TS;
    u32x4 xa[TS], xb[TS];
    // (tokens past the run's end re-read its last token: every load is
    // unconditional, and their values are not used)
#define GDN_CONV_LOAD_STAGE(xs, st)                                   \
    _Pragma("unroll") for (int u = 0; u < TS; ++u) {                  \
        const int tok = (st) * TS + u < nt ? (st) * TS + u : nt - 1; \
        xs[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xs16 + (t0 + tok) * D + c)); \
    }
    GDN_CONV_LOAD_STAGE(xa, 0)
    // taps padded at the front to four, as bf16 pairs (w~0, w~1) and (w~2, w~3)
    uint32_t w01[8], w23[8];
    {
        const uint16_t *wt = static_cast<const uint16_t *>(a.weight);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t t[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = i >= 4 - W ? wt[(c + k) * W + i - (4 - W)] : 0u;
            w01[k] = t[0] | (t[1] << 16);
            w23[k] = t[2] | (t[3] << 16);
        }
    }
    // the three positions before the run (bf16 bits): from x, from the state,
    // or zero
    auto before = [&](int back, int k) -> uint32_t {   // position t0 - back, channel c + k
        const int64_t tau = t0 - back;
        if (tau >= s0) return xs16[tau * D + c + k];
        const int64_t sb = s0 - tau;                   // 1 .. 3 positions before the start
        if (sb > P || !st16) return 0u;
        return st16[((int64_t)n * D + c + k) * P + (P - sb)];
    };
    uint32_t pm[8], pc[8];   // pairs (x[t-3], x[t-2]) and (x[t-2], x[t-1]) for the token t about to be processed
    u32x4 xp;                // x[t-1], 8 channels as 4 pairs of channels
    {
        uint32_t b3[8], b2[8], b1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            b3[k] = before(3, k);
            b2[k] = before(2, k);
            b1[k] = before(1, k);
            pm[k] = b3[k] | (b2[k] << 16);
            pc[k] = b2[k] | (b1[k] << 16);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) xp[m] = b1[2 * m] | (b1[2 * m + 1] << 16);
    }
    uint16_t *ys16 = static_cast<uint16_t *>(a.y);
#define GDN_CONV_RUN_STAGE(xs, st)                                                         \
    _Pragma("unroll") for (int u = 0; u < TS; ++u) {                                       \
        if ((st) * TS + u < nt) {                                                          \
            const u32x4 xc = xs[u];                                                        \
            uint32_t pn[8];                                                                \
            _Pragma("unroll") for (int m = 0; m < 4; ++m) {                                \
                pn[2 * m] = pair_lo(xp[m], xc[m]);                                         \
                pn[2 * m + 1] = pair_hi(xp[m], xc[m]);                                     \
            }                                                                              \
            float out[8];                                                                  \
            _Pragma("unroll") for (int k = 0; k < 8; ++k) {                                \
                const float acc = dot2bf(w23[k], pn[k], dot2bf(w01[k], pm[k], 0.f));       \
                out[k] = a.activation ? silu(acc) : acc;                                   \
            }                                                                              \
            Vec8<bf16_t>::store_nt(ys16, (t0 + (st) * TS + u) * D + c, out);               \
            _Pragma("unroll") for (int k = 0; k < 8; ++k) {                                \
                pm[k] = pc[k];                                                             \
                pc[k] = pn[k];                                                             \
            }                                                                              \
            xp = xc;                                                                       \
        }                                                                                  \
    }
    // two register sets with fixed homes: stage st in xa (st even) or xb (odd)
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst) { GDN_CONV_LOAD_STAGE(xb, st + 1) }
        GDN_CONV_RUN_STAGE(xa, st)
        if (st + 1 >= nst) break;
        if (st + 2 < nst) { GDN_CONV_LOAD_STAGE(xa, st + 2) }
        GDN_CONV_RUN_STAGE(xb, st + 1)
    }
#undef GDN_CONV_LOAD_STAGE
#undef GDN_CONV_RUN_STAGE
    if (t0 + nt == s1 && a.state_out) {
        // the run holding the sequence's last token t writes its state: positions
        // t - P + 1 .. t; pm = (x[t-2], x[t-1]) and pc = (x[t-1], x[t]) after the loop
        uint16_t *so = static_cast<uint16_t *>(a.state_out);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                if (j >= P) continue;
                const int i = 3 - P + j;   // 0: x[t-2], 1: x[t-1], 2: x[t] (no run-time array index)
                const uint32_t v = i == 0 ? pm[k] : i == 1 ? pc[k] : (pc[k] >> 16);
                so[((int64_t)n * D + c + k) * P + j] = (uint16_t)(v & 0xffffu);
            }
        }
    }
}

// Gated RMSNorm with L = V / 8 lanes per row (a power of two up to 64): each
// lane reads 8 consecutive elements of o and z in one access, so a wave covers
// 64 / L rows per pass; the row sum of squares is reduced over its L lanes.
template <typename T, int L>
__global__ __launch_bounds__(256) void gated_rmsnorm8_kernel(NormArgs a) {
    constexpr int RPW = 64 / L;   // rows per wave pass
    const int lane = threadIdx.x & 63, sub = lane % L, rl = lane / L;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t n_waves = ((int64_t)gridDim.x * 256) >> 6;
    const int V = 8 * L;
    float wt[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) wt[k] = a.weight[8 * sub + k];
    for (int64_t r0 = wave * RPW; r0 < a.rows; r0 += n_waves * RPW) {
        const int64_t r = r0 + rl;
        const bool ok = r < a.rows;
        float o[8], z[8];
        if (ok) Vec8<T>::load_nt(a.o, r * V + 8 * sub, o);
        else
#pragma unroll
            for (int k = 0; k < 8; ++k) o[k] = 0.f;
        if (ok && a.z) Vec8<T>::load_nt(a.z, r * V + 8 * sub, z);
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) ss = fmaf(o[k], o[k], ss);
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
        const float inv = rsqrtf(ss / (float)V + a.eps);
        float y[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            y[k] = o[k] * inv * wt[k];
            if (a.z) y[k] *= silu(z[k]);
        }
        if (ok) Vec8<T>::store_nt(a.y, r * V + 8 * sub, y);
    }
}

}  // namespace

hipError_t launch_causal_conv(int dtype, const ConvArgs &a, hipStream_t s) {
    if (a.D % 8 == 0) {
        // runs of kConvRun tokens, laid out sequence by sequence
        ConvArgs b = a;
        if (a.packed) {
            int64_t nb = 0;
            for (int n = 0; n < a.N; ++n) {
                b.block_start[n] = (int32_t)nb;
                nb += (a.start[n + 1] - a.start[n] + kConvRun - 1) / kConvRun;
            }
            b.block_start[a.N] = (int32_t)nb;
            b.n_blocks = nb;
        } else {
            b.n_blocks = (int64_t)a.N * ((a.S + kConvRun - 1) / kConvRun);
        }
        const int64_t groups = a.D / 8;
        b.n_cg = (int32_t)((groups + kConvThreads - 1) / kConvThreads);
        if ((b.n_blocks + 1) * b.n_cg > 0x7fffffffLL) return hipErrorInvalidConfiguration;   // grid limit
        const dim3 grid((unsigned)((b.n_blocks + 1) * b.n_cg)), block(kConvThreads);
        if (a.W <= 4) {
            if (dtype == GDN_F32) hipLaunchKernelGGL((causal_conv_run_kernel<float, 4>), grid, block, 0, s, b);
            else hipLaunchKernelGGL(causal_conv_run_bf16w4_kernel, grid, block, 0, s, b);
        } else {
            if (dtype == GDN_F32) hipLaunchKernelGGL((causal_conv_run_kernel<float, 8>), grid, block, 0, s, b);
            else hipLaunchKernelGGL((causal_conv_run_kernel<bf16_t, 8>), grid, block, 0, s, b);
        }
        return hipGetLastError();
    }
    const int64_t tblocks = (a.T + kConvTokens - 1) / kConvTokens;
    const dim3 grid((unsigned)(tblocks + 1), (unsigned)((a.D + kConvThreads - 1) / kConvThreads)), block(kConvThreads);
    if (dtype == GDN_F32) hipLaunchKernelGGL(causal_conv_kernel<float>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(causal_conv_kernel<bf16_t>, grid, block, 0, s, a);
    return hipGetLastError();
}

template <int L>
hipError_t launch_norm8(int dtype, const NormArgs &a, hipStream_t s) {
    const int64_t waves = (a.rows + 64 / L - 1) / (64 / L);
    const int64_t blocks = (waves + 3) / 4 < 8192 ? (waves + 3) / 4 : 8192;
    if (dtype == GDN_F32) hipLaunchKernelGGL((gated_rmsnorm8_kernel<float, L>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gated_rmsnorm8_kernel<bf16_t, L>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(int dtype, const NormArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    switch (a.V) {
        case 8: return launch_norm8<1>(dtype, a, s);
        case 16: return launch_norm8<2>(dtype, a, s);
        case 32: return launch_norm8<4>(dtype, a, s);
        case 64: return launch_norm8<8>(dtype, a, s);
        case 128: return launch_norm8<16>(dtype, a, s);
        case 256: return launch_norm8<32>(dtype, a, s);
        default: break;
    }
    const int64_t waves = a.rows;
    const int64_t blocks = (waves + 3) / 4 < 4096 ? (waves + 3) / 4 : 4096;
    if (blocks == 0) return hipSuccess;
    if (dtype == GDN_F32) hipLaunchKernelGGL(gated_rmsnorm_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(gated_rmsnorm_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace gdn
