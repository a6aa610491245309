// qknr.hip -- fused per-head QK-Norm + RoPE for AMD MI355X (gfx950, CDNA4).
//
// The operation (RMSNorm with a static weight and a per-row inverse-RMS
// scalar, as decomposed in the abstract of "QK-Normed MLA: QK normalization
// without full key caching"; applied per head as in the QG-MIL and HobbyLM
// abstracts; then RoPE on the first rotary_dim channels, "Fractional Rotation,
// Full Potential? Investigating Performance and Convergence of Partial RoPE",
// abstract) is fused into one pass over HBM in each direction, the "QK-RoPE"
// fusion of the Chronicals abstract, contribution (1).
//
// The path is bound by HBM bandwidth (a few fp32 operations per byte), so it
// uses no matrix cores.  Design, per launch:
//   * A workgroup of 256 threads (4 wave64) owns tiles of 16 consecutive
//     tokens.  For a tile it first evaluates cos/sin of pos * theta_i in fp64
//     (rounded to fp32) once per (token, frequency) into LDS; every Q and K row
//     of those tokens then reads them from LDS.  No cos/sin table in HBM.
//   * A row (one head vector) is spread over L = head_dim / (2 * E) lanes,
//     E elements per 16-byte chunk (8 for bf16, 4 for fp32).  Each lane loads
//     two 16-byte chunks chosen so that every RoPE pair (i, i + R/2) sits in
//     the same lane: lane j < R/(2E) holds chunks j and j + R/(2E); the other
//     lanes hold two adjacent unrotated chunks.  The rotation never crosses
//     lanes; only the row sums (sum x^2, and in the backward sum u*xh) are
//     reduced across the L lanes, with DPP adds.
//   * The tile's Q rows and K rows are each a contiguous block of memory.  A
//     wave owns groups of 64/L rows that are all Q or all K, so per-group
//     choices (weights, which dw accumulator) are wave-uniform.
//   * Loads for a batch of groups are issued before any arithmetic on them.
//   * Backward: dw is accumulated per lane in fp32 registers over all rows a
//     workgroup processes, reduced through LDS in a fixed order into one
//     partial per workgroup, and summed over workgroups in a fixed order by a
//     small second kernel: bit-reproducible, no atomics.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include "qknr.h"

namespace {

constexpr int kThreads = 256;            // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kTileTokens = 16;          // tokens per tile (multiple of every rows-per-wave)
constexpr int kMaxHeadDim = 256;
constexpr int kMaxHalf = kMaxHeadDim / 2;
constexpr int kMaxHeads = 1024;          // bound for the float-reciprocal row -> token division
constexpr int kMaxBwdBlocks = 512;       // partial-sum slots for dw (workgroups of the backward)
constexpr int kFinalizeThreads = 1024;
constexpr int kFinalizeCols = 64;

struct Bf16 {      // bf16 storage element (bit pattern); pointer arithmetic on
    uint16_t bits; // Bf16* steps by 2 bytes
};

template <typename IO> struct Io;

template <> struct Io<float> {
    static constexpr int E = 4;
    __device__ static inline void unpack(const uint4 v, float *f)
    {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    __device__ static inline uint4 pack(const float *f)
    {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
    __device__ static inline void store_scalar(void *p, int64_t i, float v)
    {
        static_cast<float *>(p)[i] = v;
    }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 pair -> bf16 pair (one v_cvt_pk_bf16_f32 on gfx950).
__device__ inline uint32_t pack_bf16x2(float lo, float hi)
{
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <> struct Io<Bf16> {
    static constexpr int E = 8;
    __device__ static inline void unpack(const uint4 v, float *f)
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static inline uint4 pack(const float *f)
    {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
    __device__ static inline void store_scalar(void *p, int64_t i, float v)
    {
        f32x2_t x = {v, 0.0f};
        bf16x2_t b = __builtin_convertvector(x, bf16x2_t);
        static_cast<__bf16 *>(p)[i] = b[0];
    }
};

__device__ inline uint4 ld16(const void *p) { return *static_cast<const uint4 *>(p); }
__device__ inline void st16(void *p, uint4 v) { *static_cast<uint4 *>(p) = v; }

// Sum over aligned groups of L lanes; every lane of a group gets the total.
// Steps: xor 1 and xor 2 inside quads, then half-row and row mirrors (lane i
// pairs with 7-i, then 15-i), then a swap of 16-lane halves.
template <int L> __device__ inline float group_sum(float v)
{
    static_assert(L == 2 || L == 4 || L == 8 || L == 16 || L == 32, "lanes per row");
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0xB1, 0xF, 0xF, true));
    if constexpr (L >= 4)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   0x4E, 0xF, 0xF, true));
    if constexpr (L >= 8)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   0x141, 0xF, 0xF, true));
    if constexpr (L >= 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   0x140, 0xF, 0xF, true));
    if constexpr (L >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                   0x401F));
    return v;
}

struct Params {
    const void *x[2];        // q, k
    const void *dy[2];       // dq_out, dk_out (backward only)
    void *out[2];            // q_out, k_out (forward) or dq, dk (backward)
    const void *w[2];        // wq, wk
    const int32_t *pos;
    float *partials;         // [gridDim.x][2][D] (backward only)
    int64_t tokens;
    int32_t heads[2];        // hq, hkv
    int32_t rotary_dim;
    float eps;
    float inv_heads[2];      // 1.0f / heads (row -> token division)
    int64_t tiles;
    double inv_freq[kMaxHalf];  // theta^(-2i/R), computed on the host in fp64
};

// Per-lane layout of a row: which two chunks this lane holds and whether they
// form RoPE pairs.
template <typename IO, int D> struct Lane {
    static constexpr int E = Io<IO>::E;
    static_assert(sizeof(IO) * E == 16, "a chunk is 16 bytes of storage elements");
    static constexpr int C = D / E;     // 16-byte chunks per row
    static constexpr int L = C / 2;     // lanes per row
    static constexpr int RW = 64 / L;   // rows per wave per group
    static_assert(kTileTokens % RW == 0, "tile must hold whole groups of every segment");
    int j;       // lane within row
    int rho;     // row within group
    int ca, cb;  // chunk indices
    bool rot;
    __device__ Lane(int lane, int rotary_dim)
    {
        j = lane % L;
        rho = lane / L;
        const int hc = (rotary_dim / 2) / E;  // lanes that hold RoPE pairs
        rot = j < hc;
        ca = rot ? j : 2 * hc + 2 * (j - hc);
        cb = rot ? j + hc : ca + 1;
    }
};

// Fill the tile's cos/sin table: cs[tl * kMaxHalf... ] laid out [token][i].
// Values are cos/sin of pos * inv_freq[i] in fp64, rounded to fp32.
template <int D>
__device__ inline void fill_cos_sin(const Params &p, int64_t tok0, float2 *cs)
{
    const int h = p.rotary_dim >> 1;
    const int n = kTileTokens * h;
    for (int e = threadIdx.x; e < n; e += kThreads) {
        const int tl = e / h;
        const int i = e - tl * h;
        const int64_t t = tok0 + tl;
        float2 v = make_float2(1.0f, 0.0f);
        if (t < p.tokens) {
            const double phi = (double)p.pos[t] * p.inv_freq[i];
            double sn, cn;
            sincos(phi, &sn, &cn);
            v = make_float2((float)cn, (float)sn);
        }
        cs[tl * (D / 2) + i] = v;
    }
}

// Where group g of the tile lives.  Returns false for rows past the end.
struct RowRef {
    int64_t elem;  // element offset of the row in its tensor
    int seg;       // 0 = Q, 1 = K
    int tl;        // token within the tile
    bool valid;
};

template <int D, int RW>
__device__ inline RowRef locate(const Params &p, int64_t tok0, int nt, int gq, int g, int rho)
{
    RowRef r;
    const int seg = g < gq ? 0 : 1;
    const int gl = seg ? g - gq : g;
    const int H = p.heads[seg];
    const int rr = gl * RW + rho;  // row within the tile's segment block
    // rr < 16 * 1024 and H <= 1024: the rounded reciprocal cannot move
    // (rr + 0.5) / H across an integer.
    int tl = __float2int_rz(((float)rr + 0.5f) * p.inv_heads[seg]);
    r.valid = rr < nt * H;
    r.tl = tl < kTileTokens ? tl : kTileTokens - 1;
    r.seg = seg;
    r.elem = (tok0 * H + rr) * (int64_t)D;
    return r;
}

template <typename IO, int D, int U>
__global__ __launch_bounds__(kThreads) void qknr_fwd_kernel(const Params p)
{
    using IOT = Io<IO>;
    using LN = Lane<IO, D>;
    constexpr int E = LN::E, L = LN::L, RW = LN::RW;
    __shared__ float4 cs4[kTileTokens * (D / 2) / 2];
    float2 *cs = reinterpret_cast<float2 *>(cs4);

    const int wave = threadIdx.x >> 6;
    const LN ln(threadIdx.x & 63, p.rotary_dim);
    const int64_t tok0 = (int64_t)blockIdx.x * kTileTokens;
    const int64_t left = p.tokens - tok0;
    const int nt = left < kTileTokens ? (int)left : kTileTokens;
    const int gq = kTileTokens * p.heads[0] / RW;
    const int G = gq + kTileTokens * p.heads[1] / RW;

    float w[2][2][E];  // [seg][chunk a/b][e]
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        IOT::unpack(ld16(static_cast<const char *>(p.w[s]) + ln.ca * 16), w[s][0]);
        IOT::unpack(ld16(static_cast<const char *>(p.w[s]) + ln.cb * 16), w[s][1]);
    }

    uint4 va[U], vb[U];
    RowRef rr[U];
    auto issue = [&](int g0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u * kWaves;
            rr[u] = locate<D, RW>(p, tok0, nt, gq, g < G ? g : G - 1, ln.rho);
            rr[u].valid = rr[u].valid && g < G;
            va[u] = make_uint4(0, 0, 0, 0);
            vb[u] = make_uint4(0, 0, 0, 0);
            if (rr[u].valid) {
                const IO *base = static_cast<const IO *>(p.x[rr[u].seg]) + rr[u].elem;
                va[u] = ld16(base + ln.ca * E);
                vb[u] = ld16(base + ln.cb * E);
            }
        }
    };

    int g0 = wave;
    issue(g0);
    fill_cos_sin<D>(p, tok0, cs);
    __syncthreads();

    const float eps = p.eps;
    constexpr float inv_d = 1.0f / D;
    for (;;) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float xa[E], xb[E];
            IOT::unpack(va[u], xa);
            IOT::unpack(vb[u], xb);
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                ss = fmaf(xa[e], xa[e], fmaf(xb[e], xb[e], ss));
            ss = group_sum<L>(ss);
            const float r = rsqrtf(fmaf(ss, inv_d, eps));
            float wa[E], wb[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                wa[e] = rr[u].seg ? w[1][0][e] : w[0][0][e];
                wb[e] = rr[u].seg ? w[1][1][e] : w[0][1][e];
            }
            float c[E], s[E];
            if (ln.rot) {
                const float4 *src = reinterpret_cast<const float4 *>(cs + rr[u].tl * (D / 2) + ln.j * E);
#pragma unroll
                for (int e = 0; e < E / 2; ++e) {
                    const float4 v = src[e];
                    c[2 * e] = v.x;
                    s[2 * e] = v.y;
                    c[2 * e + 1] = v.z;
                    s[2 * e + 1] = v.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    c[e] = 1.0f;
                    s[e] = 0.0f;
                }
            }
            float ya[E], yb[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float na = xa[e] * r * wa[e];
                const float nb = xb[e] * r * wb[e];
                ya[e] = fmaf(na, c[e], -nb * s[e]);
                yb[e] = fmaf(nb, c[e], na * s[e]);
            }
            if (rr[u].valid) {
                IO *base = static_cast<IO *>(p.out[rr[u].seg]) + rr[u].elem;
                st16(base + ln.ca * E, IOT::pack(ya));
                st16(base + ln.cb * E, IOT::pack(yb));
            }
        }
        g0 += U * kWaves;
        if (g0 >= G)
            break;
        issue(g0);
    }
}

template <typename IO, int D, int U>
__global__ __launch_bounds__(kThreads) void qknr_bwd_kernel(const Params p)
{
    using IOT = Io<IO>;
    using LN = Lane<IO, D>;
    constexpr int E = LN::E, L = LN::L, RW = LN::RW;
    constexpr int kCsFloats = kTileTokens * (D / 2) * 2;
    constexpr int kRedFloats = kWaves * RW * D;
    constexpr int kSmem = kCsFloats > kRedFloats ? kCsFloats : kRedFloats;
    __shared__ float4 smem4[kSmem / 4];
    float2 *cs = reinterpret_cast<float2 *>(smem4);
    float *red = reinterpret_cast<float *>(smem4);

    const int wave = threadIdx.x >> 6;
    const LN ln(threadIdx.x & 63, p.rotary_dim);
    const int gq = kTileTokens * p.heads[0] / RW;
    const int G = gq + kTileTokens * p.heads[1] / RW;

    float w[2][2][E];
    float acc[2][2][E];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        IOT::unpack(ld16(static_cast<const char *>(p.w[s]) + ln.ca * 16), w[s][0]);
        IOT::unpack(ld16(static_cast<const char *>(p.w[s]) + ln.cb * 16), w[s][1]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            acc[s][0][e] = 0.0f;
            acc[s][1][e] = 0.0f;
        }
    }

    const float eps = p.eps;
    constexpr float inv_d = 1.0f / D;

    for (int64_t tile = blockIdx.x; tile < p.tiles; tile += gridDim.x) {
        const int64_t tok0 = tile * kTileTokens;
        const int64_t left = p.tokens - tok0;
        const int nt = left < kTileTokens ? (int)left : kTileTokens;

        uint4 xa4[U], xb4[U], da4[U], db4[U];
        RowRef rr[U];
        auto issue = [&](int g0) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int g = g0 + u * kWaves;
                rr[u] = locate<D, RW>(p, tok0, nt, gq, g < G ? g : G - 1, ln.rho);
                rr[u].valid = rr[u].valid && g < G;
                xa4[u] = xb4[u] = da4[u] = db4[u] = make_uint4(0, 0, 0, 0);
                if (rr[u].valid) {
                    const IO *xb = static_cast<const IO *>(p.x[rr[u].seg]) + rr[u].elem;
                    const IO *db = static_cast<const IO *>(p.dy[rr[u].seg]) + rr[u].elem;
                    xa4[u] = ld16(xb + ln.ca * E);
                    xb4[u] = ld16(xb + ln.cb * E);
                    da4[u] = ld16(db + ln.ca * E);
                    db4[u] = ld16(db + ln.cb * E);
                }
            }
        };

        int g0 = wave;
        issue(g0);
        __syncthreads();  // previous tile's readers of cs are done
        fill_cos_sin<D>(p, tok0, cs);
        __syncthreads();

        for (;;) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float xa[E], xb[E], ga[E], gb[E];
                IOT::unpack(xa4[u], xa);
                IOT::unpack(xb4[u], xb);
                IOT::unpack(da4[u], ga);
                IOT::unpack(db4[u], gb);
                float ss = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    ss = fmaf(xa[e], xa[e], fmaf(xb[e], xb[e], ss));
                ss = group_sum<L>(ss);
                const float r = rsqrtf(fmaf(ss, inv_d, eps));
                if (ln.rot) {
                    // g = R^T dy: rotate the upstream gradient by -phi.
                    const float4 *src = reinterpret_cast<const float4 *>(cs + rr[u].tl * (D / 2) + ln.j * E);
#pragma unroll
                    for (int e = 0; e < E / 2; ++e) {
                        const float4 v = src[e];
                        const float c0 = v.x, s0 = v.y, c1 = v.z, s1 = v.w;
                        const float a0 = ga[2 * e], b0 = gb[2 * e];
                        const float a1 = ga[2 * e + 1], b1 = gb[2 * e + 1];
                        ga[2 * e] = fmaf(a0, c0, b0 * s0);
                        gb[2 * e] = fmaf(b0, c0, -a0 * s0);
                        ga[2 * e + 1] = fmaf(a1, c1, b1 * s1);
                        gb[2 * e + 1] = fmaf(b1, c1, -a1 * s1);
                    }
                }
                const int sg = rr[u].seg;
                float wa[E], wb[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    wa[e] = sg ? w[1][0][e] : w[0][0][e];
                    wb[e] = sg ? w[1][1][e] : w[0][1][e];
                }
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    xa[e] *= r;  // xh
                    xb[e] *= r;
                    dot = fmaf(wa[e] * ga[e], xa[e], fmaf(wb[e] * gb[e], xb[e], dot));
                }
                dot = group_sum<L>(dot);
                const float mean = dot * inv_d;
                float da[E], db[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    da[e] = r * fmaf(-xa[e], mean, wa[e] * ga[e]);
                    db[e] = r * fmaf(-xb[e], mean, wb[e] * gb[e]);
                }
                if (sg == 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        acc[0][0][e] = fmaf(ga[e], xa[e], acc[0][0][e]);
                        acc[0][1][e] = fmaf(gb[e], xb[e], acc[0][1][e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        acc[1][0][e] = fmaf(ga[e], xa[e], acc[1][0][e]);
                        acc[1][1][e] = fmaf(gb[e], xb[e], acc[1][1][e]);
                    }
                }
                if (rr[u].valid) {
                    IO *base = static_cast<IO *>(p.out[sg]) + rr[u].elem;
                    st16(base + ln.ca * E, IOT::pack(da));
                    st16(base + ln.cb * E, IOT::pack(db));
                }
            }
            g0 += U * kWaves;
            if (g0 >= G)
                break;
            issue(g0);
        }
    }

    // Fixed-order reduction of the per-lane dw accumulators: LDS [slot][D],
    // slot = wave * RW + row-in-group, then one thread per channel sums the
    // slots in order.
    const int slot = wave * RW + ln.rho;
    float *part = p.partials + (int64_t)blockIdx.x * 2 * D;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
            red[slot * D + ln.ca * E + e] = acc[s][0][e];
            red[slot * D + ln.cb * E + e] = acc[s][1][e];
        }
        __syncthreads();
        for (int c = threadIdx.x; c < D; c += kThreads) {
            float t = 0.0f;
            for (int k = 0; k < kWaves * RW; ++k)
                t += red[k * D + c];
            part[s * D + c] = t;
        }
    }
}

// dw[c] = sum over workgroups b = 0..P-1 of partials[b][c], in a fixed order:
// 16 interleaved running sums per column, then combined in index order.
template <typename IO>
__global__ __launch_bounds__(kFinalizeThreads) void qknr_dw_finalize_kernel(
    const float *__restrict__ partials, int P, int D, void *dwq, void *dwk)
{
    constexpr int kPhases = kFinalizeThreads / kFinalizeCols;
    __shared__ float sums[kPhases][kFinalizeCols];
    const int c = blockIdx.x * kFinalizeCols + (threadIdx.x % kFinalizeCols);
    const int ph = threadIdx.x / kFinalizeCols;
    const int D2 = 2 * D;
    float t = 0.0f;
    if (c < D2)
        for (int b = ph; b < P; b += kPhases)
            t += partials[(int64_t)b * D2 + c];
    sums[ph][threadIdx.x % kFinalizeCols] = t;
    __syncthreads();
    if (ph == 0 && c < D2) {
        float s = 0.0f;
        for (int k = 0; k < kPhases; ++k)
            s += sums[k][threadIdx.x];
        if (c < D)
            Io<IO>::store_scalar(dwq, c, s);
        else
            Io<IO>::store_scalar(dwk, c - D, s);
    }
}

__global__ __launch_bounds__(256) void qknr_copy_kernel(const uint4 *__restrict__ src,
                                                        uint4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

__global__ __launch_bounds__(256) void qknr_flush_kernel(uint4 *__restrict__ buf, int64_t n,
                                                         uint32_t seed)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const uint32_t v = (uint32_t)i ^ seed;
        buf[i] = make_uint4(v, v + 1, v + 2, v + 3);
    }
}

// ---- host side ---------------------------------------------------------------

constexpr int kFwdUnroll = 4;
constexpr int kBwdUnroll = 2;

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int elem_bytes(qknr_dtype dt) { return dt == QKNR_BF16 ? 2 : 4; }

int64_t num_tiles(int64_t tokens) { return (tokens + kTileTokens - 1) / kTileTokens; }

int64_t bwd_blocks(int64_t tokens)
{
    const int64_t t = num_tiles(tokens);
    return t < kMaxBwdBlocks ? t : kMaxBwdBlocks;
}

qknr_status check_common(const void *q, const void *k, const void *wq, const void *wk,
                         const int32_t *pos, int64_t tokens, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                         qknr_dtype dtype)
{
    if (tokens < 0 || hq < 1 || hkv < 1 || hq > kMaxHeads || hkv > kMaxHeads)
        return QKNR_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps) || !(theta > 0.0) || !isfinite(theta))
        return QKNR_ERR_INVALID_ARG;
    if (dtype != QKNR_F32 && dtype != QKNR_BF16)
        return QKNR_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return QKNR_ERR_UNSUPPORTED;
    if (rotary_dim < 0 || rotary_dim > head_dim || rotary_dim % 16 != 0)
        return QKNR_ERR_UNSUPPORTED;
    if (tokens > ((int64_t)1 << 40))
        return QKNR_ERR_INVALID_ARG;
    if (tokens == 0)
        return QKNR_OK;
    if (!q || !k || !wq || !wk || !pos)
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(wq, 16) || !aligned(wk, 16) ||
        !aligned(pos, 4))
        return QKNR_ERR_MISALIGNED;
    return QKNR_OK;
}

void fill_params(Params &p, const void *q, const void *k, const void *wq, const void *wk,
                 const int32_t *pos, int64_t tokens, int32_t hq, int32_t hkv,
                 int32_t rotary_dim, float eps, double theta)
{
    memset(&p, 0, sizeof p);
    p.x[0] = q;
    p.x[1] = k;
    p.w[0] = wq;
    p.w[1] = wk;
    p.pos = pos;
    p.tokens = tokens;
    p.heads[0] = hq;
    p.heads[1] = hkv;
    p.inv_heads[0] = 1.0f / (float)hq;
    p.inv_heads[1] = 1.0f / (float)hkv;
    p.rotary_dim = rotary_dim;
    p.eps = eps;
    p.tiles = num_tiles(tokens);
    // RoPE frequencies theta^(-2i/R) in fp64 (Rope to Nope and Back Again,
    // abstract: RoPE; exponent over the rotated width R, Partial RoPE abstract).
    for (int i = 0; i < rotary_dim / 2; ++i)
        p.inv_freq[i] = pow(theta, -2.0 * (double)i / (double)rotary_dim);
}

template <typename IO, int D>
hipError_t launch_fwd(const Params &p, hipStream_t s)
{
    hipLaunchKernelGGL((qknr_fwd_kernel<IO, D, kFwdUnroll>), dim3((unsigned)p.tiles),
                       dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename IO, int D>
hipError_t launch_bwd(const Params &p, int64_t blocks, void *dwq, void *dwk, hipStream_t s)
{
    hipLaunchKernelGGL((qknr_bwd_kernel<IO, D, kBwdUnroll>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int cols = 2 * D;
    hipLaunchKernelGGL((qknr_dw_finalize_kernel<IO>),
                       dim3((cols + kFinalizeCols - 1) / kFinalizeCols), dim3(kFinalizeThreads),
                       0, s, (const float *)p.partials, (int)blocks, D, dwq, dwk);
    return hipGetLastError();
}

}  // namespace

extern "C" {

const char *qknr_status_string(qknr_status s)
{
    switch (s) {
    case QKNR_OK: return "ok";
    case QKNR_ERR_INVALID_ARG: return "invalid argument";
    case QKNR_ERR_UNSUPPORTED: return "unsupported head_dim, rotary_dim or dtype";
    case QKNR_ERR_MISALIGNED: return "pointer not aligned (tensors 16 bytes, positions 4 bytes)";
    case QKNR_ERR_WORKSPACE: return "workspace missing or too small";
    case QKNR_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

qknr_status qknr_fwd(const void *q, const void *k, const void *wq, const void *wk,
                     const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                     int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                     qknr_dtype dtype, void *q_out, void *k_out, void *stream)
{
    qknr_status st = check_common(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim,
                                  rotary_dim, eps, theta, dtype);
    if (st != QKNR_OK || tokens == 0)
        return st;
    if (!q_out || !k_out)
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(q_out, 16) || !aligned(k_out, 16))
        return QKNR_ERR_MISALIGNED;
    Params p;
    fill_params(p, q, k, wq, wk, position_ids, tokens, hq, hkv, rotary_dim, eps, theta);
    p.out[0] = q_out;
    p.out[1] = k_out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == QKNR_BF16) {
        e = head_dim == 64 ? launch_fwd<Bf16, 64>(p, s)
          : head_dim == 128 ? launch_fwd<Bf16, 128>(p, s) : launch_fwd<Bf16, 256>(p, s);
    } else {
        e = head_dim == 64 ? launch_fwd<float, 64>(p, s)
          : head_dim == 128 ? launch_fwd<float, 128>(p, s) : launch_fwd<float, 256>(p, s);
    }
    return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

size_t qknr_bwd_workspace_bytes(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                                qknr_dtype dtype)
{
    (void)hq;
    (void)hkv;
    (void)dtype;
    if (tokens <= 0 || (head_dim != 64 && head_dim != 128 && head_dim != 256))
        return 0;
    return (size_t)bwd_blocks(tokens) * 2 * (size_t)head_dim * sizeof(float);
}

qknr_status qknr_bwd(const void *q, const void *k, const void *wq, const void *wk,
                     const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                     int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                     qknr_dtype dtype, const void *dq_out, const void *dk_out, void *dq,
                     void *dk, void *dwq, void *dwk, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    qknr_status st = check_common(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim,
                                  rotary_dim, eps, theta, dtype);
    if (st != QKNR_OK || tokens == 0)
        return st;
    if (!dq_out || !dk_out || !dq || !dk || !dwq || !dwk)
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(dq_out, 16) || !aligned(dk_out, 16) || !aligned(dq, 16) || !aligned(dk, 16) ||
        !aligned(dwq, 16) || !aligned(dwk, 16))
        return QKNR_ERR_MISALIGNED;
    const size_t need = qknr_bwd_workspace_bytes(tokens, hq, hkv, head_dim, dtype);
    if (!workspace || workspace_bytes < need)
        return QKNR_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return QKNR_ERR_MISALIGNED;
    Params p;
    fill_params(p, q, k, wq, wk, position_ids, tokens, hq, hkv, rotary_dim, eps, theta);
    p.dy[0] = dq_out;
    p.dy[1] = dk_out;
    p.out[0] = dq;
    p.out[1] = dk;
    p.partials = static_cast<float *>(workspace);
    const int64_t blocks = bwd_blocks(tokens);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == QKNR_BF16) {
        e = head_dim == 64 ? launch_bwd<Bf16, 64>(p, blocks, dwq, dwk, s)
          : head_dim == 128 ? launch_bwd<Bf16, 128>(p, blocks, dwq, dwk, s)
                            : launch_bwd<Bf16, 256>(p, blocks, dwq, dwk, s);
    } else {
        e = head_dim == 64 ? launch_bwd<float, 64>(p, blocks, dwq, dwk, s)
          : head_dim == 128 ? launch_bwd<float, 128>(p, blocks, dwq, dwk, s)
                            : launch_bwd<float, 256>(p, blocks, dwq, dwk, s);
    }
    return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

qknr_status qknr_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0)
        return QKNR_OK;
    if (!src || !dst)
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(src, 16) || !aligned(dst, 16) || bytes % 16 != 0)
        return QKNR_ERR_MISALIGNED;
    const int64_t n = (int64_t)(bytes / 16);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    hipLaunchKernelGGL(qknr_copy_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(src),
                       static_cast<uint4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

qknr_status qknr_flush(void *buf, size_t bytes, uint32_t seed, void *stream)
{
    if (bytes == 0)
        return QKNR_OK;
    if (!buf)
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(buf, 16) || bytes % 16 != 0)
        return QKNR_ERR_MISALIGNED;
    const int64_t n = (int64_t)(bytes / 16);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 256 * 64)
        blocks = 256 * 64;
    hipLaunchKernelGGL(qknr_flush_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<uint4 *>(buf), n, seed);
    return hipGetLastError() == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

}  // extern "C"
