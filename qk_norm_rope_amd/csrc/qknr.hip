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
// uses no matrix cores.  Design:
//   * Rows are taken token-major: the rows of token t are its hq Q heads then
//     its hkv K heads.  A wave processes "token blocks" of TB whole tokens and
//     evaluates the cos/sin of those tokens itself, once per (token,
//     frequency), in fp64 rounded to fp32, into a wave-private LDS table.  No
//     cos/sin table in HBM and no barrier between waves.
//   * A row (one head vector) is spread over C = head_dim / E lanes, one
//     16-byte chunk per lane (E = 8 bf16 or 4 fp32 elements), so a group of
//     64 / C rows fills a wave and one load instruction covers whole rows.
//     For half-split pairs (i, i + R/2) the chunks are placed so that the two
//     halves of every pair sit in mirrored lanes (i and C-1-i), exchanged with
//     one DPP / swizzle / permute per value; for interleaved pairs (2i, 2i+1)
//     both members sit in one lane.  Row sums (sum x^2, and in the backward
//     sum u * xh) are reduced across the C lanes with DPP adds.
//   * Rows are addressed by token stride, so Q and K may be views of a fused
//     projection output (in place); the forward can write K rows through a
//     per-token slot map (paged KV cache).
//   * Software pipeline: the loads of the next batch of groups (and the next
//     token block's positions) are in flight while the current batch is
//     computed; load counts never depend on the data.  Waves are persistent
//     over a grid-stride of token blocks.
//   * Backward: dw is accumulated per lane in fp32 registers over every row a
//     workgroup processes, reduced through LDS in a fixed order into one
//     partial per workgroup, and summed over workgroups in a fixed order by a
//     small second kernel: bit-reproducible, no atomics.
#include <hip/hip_runtime.h>

#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "qknr.h"

namespace {

constexpr int kThreads = 256;            // 4 wave64 per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kMaxHeadDim = 256;
constexpr int kMaxHalf = kMaxHeadDim / 2;
constexpr int kMaxHeads = 1024;          // bound for the float-reciprocal row -> token division
// Tuning knobs (launch shape only; every configuration computes the same result).
#ifndef QKNR_MAX_FWD_BLOCKS
#define QKNR_MAX_FWD_BLOCKS 2048
#endif
#ifndef QKNR_MAX_BWD_BLOCKS
#define QKNR_MAX_BWD_BLOCKS 512
#endif
#ifndef QKNR_FWD_UNROLL
#define QKNR_FWD_UNROLL 2
#endif
#ifndef QKNR_BWD_UNROLL
#define QKNR_BWD_UNROLL 2
#endif
#ifndef QKNR_FWD_WAVES_PER_SIMD
#define QKNR_FWD_WAVES_PER_SIMD 4
#endif
#ifndef QKNR_BWD_WAVES_PER_SIMD
#define QKNR_BWD_WAVES_PER_SIMD 2
#endif
#ifndef QKNR_MIN_COS_SIN_PER_BLOCK
#define QKNR_MIN_COS_SIN_PER_BLOCK 64
#endif
constexpr int kMaxFwdBlocks = QKNR_MAX_FWD_BLOCKS;  // forward workgroups (persistent, grid-stride)
constexpr int kMaxBwdBlocks = QKNR_MAX_BWD_BLOCKS;  // backward workgroups = dw partial-sum slots
constexpr int kFinalizeThreads = 256;   // one wave per dw column
static_assert(kMaxBwdBlocks % 64 == 0, "finalize rows per lane");
constexpr int kFwdUnroll = QKNR_FWD_UNROLL;         // groups per pipeline stage
constexpr int kBwdUnroll = QKNR_BWD_UNROLL;

struct Bf16 {      // bf16 storage element (bit pattern); pointer arithmetic on
    uint16_t bits; // Bf16* steps by 2 bytes
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename IO> struct Io;

template <> struct Io<float> {
    static constexpr int E = 4;
    __device__ static inline void unpack(const u32x4 v, float *f)
    {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    __device__ static inline u32x4 pack(const float *f)
    {
        u32x4 r = {__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                   __float_as_uint(f[3])};
        return r;
    }
    __device__ static inline void store_scalar(void *p, int64_t i, float v)
    {
        static_cast<float *>(p)[i] = v;
    }
    __device__ static inline float load_scalar(const void *p, int64_t i)
    {
        return static_cast<const float *>(p)[i];
    }
    // an element's bits, converted later by from_raw (a load whose value is
    // not used at once is not waited for at once)
    __device__ static inline uint32_t load_raw(const void *p, int64_t i)
    {
        return static_cast<const uint32_t *>(p)[i];
    }
    __device__ static inline float from_raw(uint32_t r) { return __uint_as_float(r); }
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
    __device__ static inline void unpack(const u32x4 v, float *f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    __device__ static inline u32x4 pack(const float *f)
    {
        u32x4 r = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7])};
        return r;
    }
    __device__ static inline void store_scalar(void *p, int64_t i, float v)
    {
        f32x2_t x = {v, 0.0f};
        bf16x2_t b = __builtin_convertvector(x, bf16x2_t);
        static_cast<__bf16 *>(p)[i] = b[0];
    }
    __device__ static inline float load_scalar(const void *p, int64_t i)
    {
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
    }
    __device__ static inline uint32_t load_raw(const void *p, int64_t i)
    {
        return static_cast<const uint16_t *>(p)[i];
    }
    __device__ static inline float from_raw(uint32_t r) { return __uint_as_float(r << 16); }
};

// Streaming 16-byte accesses.  Every byte of the tensors is touched exactly
// once, so loads and stores are marked non-temporal.
#ifndef QKNR_NT_LOADS
#define QKNR_NT_LOADS 1
#endif
#ifndef QKNR_NT_STORES
#define QKNR_NT_STORES 1
#endif
__device__ inline u32x4 ld16(const void *p)
{
#if QKNR_NT_LOADS
    return __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
#else
    return *static_cast<const u32x4 *>(p);
#endif
}
__device__ inline void st16(void *p, u32x4 v)
{
#if QKNR_NT_STORES
    __builtin_nontemporal_store(v, static_cast<u32x4 *>(p));
#else
    *static_cast<u32x4 *>(p) = v;
#endif
}
__device__ inline u32x4 ld16_cached(const void *p) { return *static_cast<const u32x4 *>(p); }

// Make this wave's LDS writes visible to its own later LDS reads (and keep the
// compiler from moving LDS accesses across the point).
__device__ inline void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Issue priority of this wave while it issues memory operations (the
// backwards, at two waves per SIMD, and the norm-group forward, at three): the
// wave about to issue the next stage's loads or a stage's stores then wins
// instruction issue over the other waves' arithmetic, so its memory operations
// leave sooner; 0 restores the default.
template <bool ON> __device__ inline void mem_priority(bool raise)
{
    if constexpr (ON) {
        if (raise)
            __builtin_amdgcn_s_setprio(2);
        else
            __builtin_amdgcn_s_setprio(0);
    }
}

struct Params {
    const void *x[2];        // q, k
    const void *dy[2];       // dq_out, dk_out (backward only)
    void *out[2];            // q_out, k_out (forward) or dq, dk (backward)
    const void *w[2];        // wq, wk (unused without weights)
    const void *b[2];        // bq, bk: biases added after the weight (forward, has_b)
    const int32_t *pos;
    const int64_t *slots;    // output row of each token's K (forward with a slot map)
    int64_t k_out_rows;      // rows of k_out with a slot map; other slots are skipped
    float *partials;         // [gridDim.x][2][D] per-workgroup dw partials (backward only)
    int64_t xs[2];           // token strides in elements: q, k
    int64_t ds[2];           // dq_out, dk_out
    int64_t os[2];           // q_out, k_out (forward) or dq, dk (backward)
    int64_t tokens;
    int64_t token_blocks;    // ceil(tokens / tb_tokens)
    int32_t heads[2];        // hq, hkv
    int32_t rows_per_token;  // hq + hkv
    float inv_rows_per_token;
    int32_t tb_tokens;       // tokens per token block
    int32_t groups;          // groups of 64/L rows per token block
    int32_t rotary_dim;
    int32_t has_w;           // 0: parameter-free norm (w = 1)
    int32_t has_b;           // forward: add b; backward: accumulate db partials
    int32_t layernorm;       // subtract the row mean before scaling (QK-LayerNorm)
    int32_t group[2];        // heads of q / k sharing one inverse RMS (norm-group kernel)
    int32_t head_w;          // weights, biases and their gradients are [H, D] (norm-group kernel)
    int32_t stages;          // wave stages per token (norm groups in waves; 1 otherwise)
    float eps;
    double attn;             // factor on cos and sin (1 = none)
    double inv_freq[kMaxHalf];  // RoPE frequencies, computed on the host in fp64
};

// The launch parameters' scalar fields (everything before the frequency
// table) take 256 bytes: four 64-byte scalar-cache lines when the arguments
// start on a line.  The kernels read one word 64 bytes apart from each other
// together before anything else, so the first dependent reads of the fields
// hit the cache instead of missing one line after another (a hint only: any
// placement of the arguments is read correctly).
__device__ inline void touch_params(const Params &p)
{
    static_assert(offsetof(Params, inv_freq) <= 256 && offsetof(Params, b) / 64 == 1 &&
                      offsetof(Params, ds) / 64 == 2 && offsetof(Params, tb_tokens) / 64 == 3,
                  "one touched word in each of the four lines");
    const int32_t a = (int32_t)(uintptr_t)p.x[0], b = (int32_t)(uintptr_t)p.b[0];
    const int32_t c = (int32_t)p.ds[0], d = p.tb_tokens;
    asm volatile("" ::"s"(a), "s"(b), "s"(c), "s"(d));
}

template <typename IO, int D> struct Shape {
    static constexpr int E = Io<IO>::E;
    static constexpr int C = D / E;     // 16-byte chunks per row = lanes per row
    static constexpr int RW = 64 / C;   // rows per group (one group fills a wave)
    static constexpr int kCsCap = 256;  // cos/sin entries per wave: tokens * D/2 <= 256
    static constexpr int kValsPerLane = kCsCap / 64;
    static_assert(sizeof(IO) * E == 16, "a chunk is 16 bytes of storage elements");
    static_assert(C >= 8 && C <= 64, "lanes per row");
};

// Per-lane layout of a row.  Lane i (of the C lanes of a row) holds one
// 16-byte chunk.
// Half-split pairs (i, i + R/2): with hc = R / (2E) chunk pairs (a, a + hc),
//   i < hc         first-half chunk i,       partner = lane C-1-i
//   i >= C - hc    second-half chunk C-1-i+hc, partner = lane C-1-i
//   otherwise      unrotated chunk hc + i
// so every pair sits in mirrored lanes and one load instruction covers whole
// rows (full 128-byte lines).
// Interleaved pairs (2i, 2i+1): lane i holds chunk i and both members of each
// pair sit in the same lane (E is even); chunks below R rotate.
template <typename IO, int D, bool IL> struct Lane {
    using S = Shape<IO, D>;
    int rho;     // row within group
    int ch;      // chunk held
    int pc;      // RoPE pair index block: pairs pc*E .. pc*E+E-1 (half-split rotating lanes)
    bool rot;
    bool first;  // first-half chunk of a pair: y = n c - n' s; second half: + n' s
    __device__ Lane(int lane, int rotary_dim)
    {
        const int i = lane % S::C;
        rho = lane / S::C;
        if constexpr (IL) {
            ch = i;
            rot = i * S::E < rotary_dim;
            first = false;
            pc = 0;
        } else {
            const int hc = (rotary_dim / 2) / S::E;
            first = i < hc;
            const bool second = !first && i >= S::C - hc;
            pc = first ? i : (second ? S::C - 1 - i : 0);
            ch = first ? i : (second ? S::C - 1 - i + hc : hc + i);
            rot = first || second;
        }
    }
};

// Value of the mirrored lane (C-1-i within each aligned group of C lanes).
template <int C> __device__ inline uint32_t mirror(uint32_t v)
{
    if constexpr (C == 8)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true);
    else if constexpr (C == 16)
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, true);
    else if constexpr (C == 32)
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x7C1F);
    else
        return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((threadIdx.x & 63) ^ 63) << 2, (int)v);
}
template <int C> __device__ inline float mirror(float v)
{
    return __uint_as_float(mirror<C>(__float_as_uint(v)));
}

// Sum over aligned groups of C lanes; every lane of a group gets the total.
// DPP: xor 1 and xor 2 inside quads, then half-row and row mirrors (lane i
// pairs with 7-i, then 15-i); then a swap of 16-lane halves and of 32-lane
// halves.
template <int C> __device__ inline float group_sum(float v)
{
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               0x141, 0xF, 0xF, true));
    if constexpr (C >= 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                   0x140, 0xF, 0xF, true));
    if constexpr (C >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                   0x401F));
    if constexpr (C >= 64)
        v += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                           (int)((threadIdx.x & 63) ^ 32) << 2,
                                           __builtin_bit_cast(int, v)));
    return v;
}

// One row slot of a pipeline stage.
struct RowRef {
    int64_t tok;   // token index (0 for rows past the end)
    int hofs;      // element offset of the lane's chunk within its token slice
    int seg;       // 0 = Q, 1 = K
    int tl;        // token within the token block
    bool valid;
};

template <int D, int RW, int E>
// Row g * RW + rho of the token block starting at token tok0; rows past the
// block's tokens or the tensor's end, and every row of a stage past the end
// (stage_valid false), are invalid: they read their tensor's first chunk and
// are never stored.
__device__ inline RowRef locate(const Params &p, int64_t tok0, int g, int rho, int ch,
                                bool stage_valid = true)
{
    RowRef r;
    const int R = p.rows_per_token;
    const int rr = g * RW + rho;  // token-major row within the token block
    // rr < 2 * 2048 + 64 and R <= 2048: the rounded reciprocal cannot move
    // (rr + 0.5) / R across an integer.
    const int tl = __float2int_rz(((float)rr + 0.5f) * p.inv_rows_per_token);
    const int in_tok = rr - (int)__umul24((unsigned)tl, (unsigned)R);
    const int seg = in_tok >= p.heads[0] ? 1 : 0;
    const int head = seg ? in_tok - p.heads[0] : in_tok;
    const int64_t tok = tok0 + tl;
    r.valid = stage_valid && g < p.groups && tl < p.tb_tokens && tok < p.tokens;
    r.tl = r.valid ? tl : 0;
    r.seg = seg;
    r.tok = r.valid ? tok : 0;
    r.hofs = r.valid ? head * D + ch * E : 0;
    return r;
}

template <typename IO, int D, int U, bool BWD> struct Stage {
    u32x4 x[U];
    u32x4 dy[BWD ? U : 1];
    RowRef r[U];
    int32_t pos;   // position of token (lane id) of the block, lanes < tb_tokens
    int64_t slot;  // K output row of that token (slot-mapped forward only)
    int64_t tb;
    int batch;
    bool valid;
};

// Issue the loads of one stage: the positions of its token block (used when
// batch == 0), then the lane's chunk of each of its U rows (and of dy).  The
// count and order of loads never depend on the data (rows past the end, and
// stages past the end of the wave's work, read in-bounds placeholders), so the
// compiler can wait on exactly the stage it consumes while the next stage
// stays in flight.
// Rows past the end read their tensor's first chunk (always in bounds) and are
// never stored, so every stage issues the same number of loads.
template <typename IO, int D, int U, bool BWD, bool SLOT>
__device__ inline int64_t issue_positions(const Params &p, Stage<IO, D, U, BWD> &s)
{
    const int64_t tb = s.valid ? s.tb : 0;
    const int64_t tok0 = tb * p.tb_tokens;
    // one load instruction: lane t < tb_tokens fetches token t's position (and
    // output slot)
    const int l = (int)(threadIdx.x & 63);
    const int64_t t = tok0 + (l < p.tb_tokens ? l : 0);
    const int64_t tc = t < p.tokens ? t : 0;
    s.pos = p.pos[tc];
    if constexpr (SLOT) {
        // a slot outside [0, k_out_rows) writes nothing, like a negative one
        const int64_t sv = p.slots[tc];
        s.slot = sv < p.k_out_rows ? sv : -1;
    }
    return tok0;
}

template <typename IO, int D, int U, bool BWD>
__device__ inline void issue_row(const Params &p, Stage<IO, D, U, BWD> &s, int u, const RowRef &r)
{
    const IO *x0 = static_cast<const IO *>(p.x[0]);
    const IO *x1 = static_cast<const IO *>(p.x[1]);
    const IO *d0 = static_cast<const IO *>(p.dy[0]);
    const IO *d1 = static_cast<const IO *>(p.dy[1]);
    const int64_t xs0 = p.xs[0], xs1 = p.xs[1];
    const int64_t ds0 = p.ds[0], ds1 = p.ds[1];
    s.r[u] = r;
    s.x[u] = ld16((r.seg ? x1 : x0) + (r.tok * (r.seg ? xs1 : xs0) + r.hofs));
    if constexpr (BWD)
        s.dy[u] = ld16((r.seg ? d1 : d0) + (r.tok * (r.seg ? ds1 : ds0) + r.hofs));
}

template <typename IO, int D, int U, bool BWD, bool IL, bool SLOT>
__device__ inline void issue(const Params &p, Stage<IO, D, U, BWD> &s, const Lane<IO, D, IL> &ln)
{
    using S = Shape<IO, D>;
    const int64_t tok0 = issue_positions<IO, D, U, BWD, SLOT>(p, s);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const RowRef r = locate<D, S::RW, S::E>(p, tok0, s.batch * U + u, ln.rho, ln.ch, s.valid);
        issue_row(p, s, u, r);
    }
}

// issue() for a kernel whose lanes hold the same rows of every block: the
// rows located once (fixed[u], at token block 0), only the token moves.
template <typename IO, int D, int U, bool BWD, bool SLOT>
__device__ inline void issue_fixed(const Params &p, Stage<IO, D, U, BWD> &s, const RowRef *fixed)
{
    const int64_t tok0 = issue_positions<IO, D, U, BWD, SLOT>(p, s);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        RowRef r = fixed[u];
        const int64_t tok = tok0 + r.tl;
        r.valid = s.valid && r.valid && tok < p.tokens;
        r.tok = r.valid ? tok : 0;
        r.hofs = r.valid ? r.hofs : 0;
        r.tl = r.valid ? r.tl : 0;
        issue_row(p, s, u, r);
    }
}

// (a cos x, a sin x) rounded to fp32, for |x| < 2^32, evaluated in fp64:
// additive range reduction by pi/2 (Cody and Waite) with pi/2 split in two
// doubles and fused multiply-adds, so r = x - k pi/2 carries an absolute error
// near 2^-52; then the Taylor series of sin and cos on |r| <= pi/4 (truncation
// below 1e-19) in Horner form.  The fp64 result is within a few 1e-16 of the
// exact value, so its rounding to fp32 equals the rounding of the exact
// cos/sin except when the exact value lies within that distance of an fp32
// rounding boundary.  The factor a (1 unless the caller scales the rotation,
// as RoPE extensions do) multiplies in fp64 before the rounding; a = 1 is exact.
// Constants of the evaluation: 2/pi, pi/2 as head + tail, then the Taylor
// coefficients of sin (1/17! down to -1/3!) and of cos (-1/18! down to 1/4!).
__constant__ double kSinCos[19] = {
    0x1.45f306dc9c883p-1,  0x1.921fb54442d18p+0,  0x1.1a62633145c07p-54,
    0x1.952c77030ad4ap-49, -0x1.ae7f3e733b81fp-41, 0x1.6124613a86d09p-33, -0x1.ae64567f544e4p-26,
    0x1.71de3a556c734p-19, -0x1.a01a01a01a01ap-13, 0x1.1111111111111p-7,  -0x1.5555555555555p-3,
    -0x1.6827863b97d97p-53, 0x1.ae7f3e733b81fp-45, -0x1.93974a8c07c9dp-37, 0x1.1eed8eff8d898p-29,
    -0x1.27e4fb7789f5cp-22, 0x1.a01a01a01a01ap-16, -0x1.6c16c16c16c17p-10, 0x1.5555555555555p-5};

__device__ inline float2 cos_sin_f32(double x, double a)
{
    const double k = rint(x * kSinCos[0]);                 // x * 2/pi
    double r = fma(-k, kSinCos[1], x);                     // pi/2, head
    r = fma(-k, kSinCos[2], r);                            // pi/2, tail
    const double r2 = r * r;
    double ps = kSinCos[3];
#pragma unroll
    for (int i = 4; i < 11; ++i)
        ps = fma(ps, r2, kSinCos[i]);
    const double sr = fma(r * r2, ps, r);
    double pc = kSinCos[11];
#pragma unroll
    for (int i = 12; i < 19; ++i)
        pc = fma(pc, r2, kSinCos[i]);
    pc = fma(pc, r2, -0.5);                                // -1/2!
    const double cr = fma(r2, pc, 1.0);
    // x = k pi/2 + r: rotate (cos r, sin r) by the quadrant k mod 4.
    const int q = (int)(int64_t)k & 3;
    const float fs = (float)(a * sr), fc = (float)(a * cr);
    const float c = (q & 1) ? fs : fc;
    const float s = (q & 1) ? fc : fs;
    return make_float2((q == 1 || q == 2) ? -c : c, (q & 2) ? -s : s);
}

// Which cos/sin values of a token block this lane evaluates: value k is
// v = lane + 64 k, i.e. token v / h and frequency i = v mod h, packed as
// i | token << 8 | slot << 16 with slot = token D/2 + i its place in the
// table (each field < 256: h <= 128 and the block's values fit the table).
// v / h as (v + 1/2) times the rounded reciprocal of h, truncated: for
// v < 256 and h <= 128 the quotient's fraction stays at least 1/(2h) away
// from an integer, far more than the two roundings move it (checked for
// every such v and h), and it costs a few instructions instead of an
// integer division per value.
template <typename IO, int D>
__device__ inline void cos_sin_codes(int h, int nvals, int *code)
{
    using S = Shape<IO, D>;
    static_assert(S::kValsPerLane * 64 <= 256 && D / 2 <= 128, "quotients exact in fp32");
    const float inv_h = h > 0 ? 1.0f / (float)h : 0.0f;
#pragma unroll
    for (int k = 0; k < S::kValsPerLane; ++k) {
        const int v = (int)(threadIdx.x & 63) + 64 * k;
        const int tl = __float2int_rz(((float)v + 0.5f) * inv_h);
        const int i = v - tl * h;
        code[k] = v < nvals ? i | tl << 8 | (tl * (D / 2) + i) << 16 : 0;
    }
}

// cos/sin of pos * inv_freq[i] for the token block, fp64 rounded to fp32,
// into the wave's table.  Both signs are stored, (c, -s) where the lane's
// element is the first of its pair and (c, s) where it is the second, so every
// lane computes y = n c + n' s' with no per-row sign or select: half-split
// tables put (c, -s) at slot and (c, s) kCsCap later, interleaved ones at
// 2 slot and 2 slot + 1.
template <typename IO, int D, bool IL>
__device__ inline void fill_cos_sin(int32_t pos_lane, const double *freq, double attn,
                                    const int *code, int nvals, float2 *cs)
{
    using S = Shape<IO, D>;
#pragma unroll
    for (int k = 0; k < S::kValsPerLane; ++k) {
        const int v = (int)(threadIdx.x & 63) + 64 * k;
        const int i = code[k] & 0xff, tl = (code[k] >> 8) & 0xff, slot = code[k] >> 16;
        // position of this value's token, held by lane tl
        const int pos = __builtin_amdgcn_ds_bpermute(tl << 2, pos_lane);
        if (v < nvals) {
            const float2 t = cos_sin_f32((double)pos * freq[i], attn);
            cs[IL ? 2 * slot : slot] = make_float2(t.x, -t.y);
            cs[IL ? 2 * slot + 1 : S::kCsCap + slot] = t;
        }
    }
}

// IL: interleaved pairs.  SLOT: K rows are written at the row its token's slot
// names (forward only).  EXT: the norm variants chosen at run time by
// p.layernorm (subtract the row mean first) and p.has_b (biases in the forward,
// their gradients in the backward); without EXT the kernel is plain RMSNorm.
template <typename IO, int D, int U, bool BWD, bool IL, bool SLOT, bool EXT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    BWD ? QKNR_BWD_WAVES_PER_SIMD : QKNR_FWD_WAVES_PER_SIMD, 8))) void qknr_kernel(const Params p)
{
    static_assert(!(BWD && SLOT), "slot-mapped output is a forward option");
    using IOT = Io<IO>;
    using S = Shape<IO, D>;
    constexpr int E = S::E, C = S::C, RW = S::RW;
    constexpr int kCsStride = D / 2;  // frequencies per token in the cos/sin table
    // Per wave: 2 * kCsCap table entries, then E identity entries (1, 0) that
    // lanes holding unrotated chunks read instead.  Half-split: entries
    // [token][i] of (c, -s), then kCsCap later the same of (c, s).  Interleaved:
    // entries [token][2i] = (c, -s) and [token][2i+1] = (c, s), one per channel.
    constexpr int kCsWave = 2 * S::kCsCap + E;
    __shared__ float4 cs_store[kWaves * kCsWave / 2];
    constexpr int kRedFloats = BWD ? kWaves * RW * D : 4;
    __shared__ float red[kRedFloats];
    __shared__ float4 w_store[2 * D / 4];   // [seg][D] norm weights as fp32
    __shared__ float4 b_store[EXT && !BWD ? 2 * D / 4 : 1];  // [seg][D] biases as fp32
    __shared__ double freq[D / 2];          // theta^(-2i/R)
    float *wl = reinterpret_cast<float *>(w_store);
    touch_params(p);

    const int wave = threadIdx.x >> 6;
    float2 *cs = reinterpret_cast<float2 *>(cs_store) + wave * kCsWave;
    float2 *cs_id = cs + 2 * S::kCsCap;
    const Lane<IO, D, IL> ln(threadIdx.x & 63, p.rotary_dim);
    const int h = p.rotary_dim >> 1;
    const int nvals = p.tb_tokens * h;
    if ((threadIdx.x & 63) < E)
        cs_id[threadIdx.x & 63] = make_float2(1.0f, 0.0f);
    // This lane's E cos/sin entries for a row of token tl start at
    // cs_lane + tl * cs_tok (float4 = two entries).
    const float2 *cs_row0 = IL ? cs + ln.ch * E
                               : (ln.first ? cs : cs + S::kCsCap) + ln.pc * E;
    const float4 *cs_lane = reinterpret_cast<const float4 *>(ln.rot ? cs_row0 : cs_id);
    const int cs_tok = ln.rot ? (IL ? D / 2 : kCsStride / 2) : 0;

    // The weights, biases and frequencies for LDS are loaded into registers
    // here and written to LDS only after the first stage's loads are issued
    // (below), so the kernel's first memory latency covers them all.  The
    // loads have no branch around them (a branch would make the compiler
    // wait for the value inside it): without weights or biases they read
    // the first row of q, and the value is replaced when it is written.
    constexpr int kStaged = (2 * D + kThreads - 1) / kThreads;
    uint32_t wv[kStaged], bv[kStaged];
    {
        const void *const w0 = p.has_w ? p.w[0] : p.x[0];
        const void *const w1 = p.has_w ? p.w[1] : p.x[0];
#pragma unroll
        for (int j = 0; j < kStaged; ++j) {
            const int i = min((int)threadIdx.x + j * kThreads, 2 * D - 1);
            wv[j] = IOT::load_raw(i < D ? w0 : w1, i % D);
        }
    }
    if constexpr (EXT && !BWD) {
        const void *const b0 = p.has_b ? p.b[0] : p.x[0];
        const void *const b1 = p.has_b ? p.b[1] : p.x[0];
#pragma unroll
        for (int j = 0; j < kStaged; ++j) {
            const int i = min((int)threadIdx.x + j * kThreads, 2 * D - 1);
            bv[j] = IOT::load_raw(i < D ? b0 : b1, i % D);
        }
    }
    static_assert(D / 2 <= kThreads, "one frequency per thread");
    const double fv = (int)threadIdx.x < h ? p.inv_freq[threadIdx.x] : 0.0;

    // Fixed per lane: which (token, frequency) cos/sin values it evaluates.
    int vcode[S::kValsPerLane];
    cos_sin_codes<IO, D>(h, nvals, vcode);

    // Backward: per-lane dw accumulators for Q rows and K rows, then (EXT) db.
    constexpr int kAcc = BWD ? (EXT ? 4 : 2) : 1;
    float acc[kAcc][E];
    if constexpr (BWD) {
#pragma unroll
        for (int a = 0; a < kAcc; ++a)
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[a][e] = 0.0f;
    }
    const bool layernorm = EXT && p.layernorm;
    const bool has_b = EXT && p.has_b;

    const int nbatch = (p.groups + U - 1) / U;
    const int64_t gwave = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves;
    const float eps = p.eps;
    constexpr float inv_d = 1.0f / D;

    // Output bases and strides as scalars: selecting between kernel-argument
    // fields with a per-lane index would turn into a per-lane load.
    IO *const out0 = static_cast<IO *>(p.out[0]);
    IO *const out1 = static_cast<IO *>(p.out[1]);
    const int64_t os0 = p.os[0], os1 = p.os[1];

    // Two stages: stage k+1 is in flight while stage k is computed.  The loop
    // is unrolled by two so the stages never need copying.
    auto step = [&](Stage<IO, D, U, BWD> &st) {
            if (st.batch == 0) {
                wave_sync();  // previous token block's table reads are done
                fill_cos_sin<IO, D, IL>(st.pos, freq, p.attn, vcode, nvals, cs);
                wave_sync();
            }

    #pragma unroll
            for (int u = 0; u < U; ++u) {
                const RowRef &rr = st.r[u];
                float x[E];
                IOT::unpack(st.x[u], x);
                if (layernorm) {
                    // QK-LayerNorm: centre the row on its mean first
                    float sx = 0.0f;
    #pragma unroll
                    for (int e = 0; e < E; ++e)
                        sx += x[e];
                    const float m = group_sum<C>(sx) * inv_d;
    #pragma unroll
                    for (int e = 0; e < E; ++e)
                        x[e] -= m;
                }
                float ss = 0.0f;
    #pragma unroll
                for (int e = 0; e < E; ++e)
                    ss = fmaf(x[e], x[e], ss);
                ss = group_sum<C>(ss);
                const float r = rsqrtf(fmaf(ss, inv_d, eps));
                float w[E];
                {
                    const float4 *ws = reinterpret_cast<const float4 *>(wl + rr.seg * D + ln.ch * E);
    #pragma unroll
                    for (int e = 0; e < E / 4; ++e) {
                        const float4 a = ws[e];
                        w[4 * e] = a.x; w[4 * e + 1] = a.y; w[4 * e + 2] = a.z; w[4 * e + 3] = a.w;
                    }
                }
                // c and signed s (identity for unrotated chunks), no per-row select
                float c[E], sn[E];
                {
                    const float4 *src = cs_lane + rr.tl * cs_tok;
    #pragma unroll
                    for (int e = 0; e < E / 2; ++e) {
                        const float4 v = src[e];
                        c[2 * e] = v.x;
                        sn[2 * e] = v.y;
                        c[2 * e + 1] = v.z;
                        sn[2 * e + 1] = v.w;
                    }
                }
                // output row: the token, or for K rows its slot (negative: skip)
                int64_t orow = rr.tok;
                bool store = rr.valid;
                if constexpr (SLOT) {
                    const int src = rr.tl << 2;
                    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(
                        src, (int)(uint32_t)(uint64_t)st.slot);
                    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(
                        src, (int)(uint32_t)((uint64_t)st.slot >> 32));
                    const int64_t sl = (int64_t)(((uint64_t)hi << 32) | lo);
                    orow = rr.seg ? sl : rr.tok;
                    store = store && orow >= 0;
                }
                IO *o = (rr.seg ? out1 : out0) + (orow * (rr.seg ? os1 : os0) + rr.hofs);
                if constexpr (!BWD) {
                    // y = n c + sgn n' s, n = x r w, n' the pair partner: the
                    // mirrored lane (half-split) or the neighbouring element
                    // (interleaved)
                    float n[E], y[E];
    #pragma unroll
                    for (int e = 0; e < E; ++e)
                        n[e] = x[e] * r * w[e];
                    if (has_b) {
                        const float4 *bs = b_store + (rr.seg * D + ln.ch * E) / 4;
    #pragma unroll
                        for (int e = 0; e < E / 4; ++e) {
                            const float4 a = bs[e];
                            n[4 * e] += a.x; n[4 * e + 1] += a.y; n[4 * e + 2] += a.z; n[4 * e + 3] += a.w;
                        }
                    }
    #pragma unroll
                    for (int e = 0; e < E; ++e)
                        y[e] = fmaf(n[e], c[e], (IL ? n[e ^ 1] : mirror<C>(n[e])) * sn[e]);
                    const u32x4 packed = IOT::pack(y);
                    if (store)
                        st16(o, packed);
                } else {
                    // g = R^T dy = dy c - sgn dy' s (rotation by -phi)
                    float g[E], gp[E];
                    IOT::unpack(st.dy[u], g);
                    if constexpr (IL) {
    #pragma unroll
                        for (int e = 0; e < E; ++e)
                            gp[e] = g[e ^ 1];
                    } else {
                        u32x4 dyp;
    #pragma unroll
                        for (int i = 0; i < 4; ++i)
                            dyp[i] = mirror<C>(st.dy[u][i]);
                        IOT::unpack(dyp, gp);
                    }
    #pragma unroll
                    for (int e = 0; e < E; ++e)
                        g[e] = fmaf(g[e], c[e], -gp[e] * sn[e]);
                    float dot = 0.0f;
    #pragma unroll
                    for (int e = 0; e < E; ++e) {
                        x[e] *= r;  // xh
                        dot = fmaf(w[e] * g[e], x[e], dot);
                    }
                    dot = group_sum<C>(dot);
                    const float mean = dot * inv_d;
                    // QK-LayerNorm: the centring adds -mean(u), u = w g
                    float mu = 0.0f;
                    if (layernorm) {
                        float su = 0.0f;
    #pragma unroll
                        for (int e = 0; e < E; ++e)
                            su = fmaf(w[e], g[e], su);
                        mu = group_sum<C>(su) * inv_d;
                    }
                    float dx[E];
    #pragma unroll
                    for (int e = 0; e < E; ++e)
                        dx[e] = r * fmaf(-x[e], mean, w[e] * g[e] - mu);
                    // dw += g * xh into the accumulator of this row's tensor; rows
                    // past the end (which read placeholder data) add exact zeros.
                    const float mq = (rr.valid && rr.seg == 0) ? 1.0f : 0.0f;
                    const float mk = (rr.valid && rr.seg == 1) ? 1.0f : 0.0f;
    #pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float v = g[e] * x[e];
                        acc[0][e] = fmaf(v, mq, acc[0][e]);
                        acc[1][e] = fmaf(v, mk, acc[1][e]);
                    }
                    if constexpr (EXT) {
                        // db += g (the bias enters y after the norm)
    #pragma unroll
                        for (int e = 0; e < E; ++e) {
                            acc[2][e] = fmaf(g[e], mq, acc[2][e]);
                            acc[3][e] = fmaf(g[e], mk, acc[3][e]);
                        }
                    }
                    const u32x4 packed = IOT::pack(dx);
                    mem_priority<true>(true);
                    if (store)
                        st16(o, packed);
                    mem_priority<true>(false);
                }
            }
    };
    auto advance = [&](const Stage<IO, D, U, BWD> &from, Stage<IO, D, U, BWD> &to) {
        to.batch = from.batch + 1 < nbatch ? from.batch + 1 : 0;
        to.tb = to.batch ? from.tb : from.tb + nwaves;
        to.valid = to.tb < p.token_blocks;
        mem_priority<BWD>(true);
        issue<IO, D, U, BWD, IL, SLOT>(p, to, ln);
        mem_priority<BWD>(false);
    };
    Stage<IO, D, U, BWD> sa, sb;
    sa.tb = gwave;
    sa.batch = 0;
    sa.valid = sa.tb < p.token_blocks;
    issue<IO, D, U, BWD, IL, SLOT>(p, sa, ln);
    // the staged values to LDS (their loads are older than the stage's, so
    // this waits for them alone)
#pragma unroll
    for (int j = 0; j < kStaged; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < 2 * D) {
            wl[i] = p.has_w ? IOT::from_raw(wv[j]) : 1.0f;
            if constexpr (EXT && !BWD)
                reinterpret_cast<float *>(b_store)[i] = p.has_b ? IOT::from_raw(bv[j]) : 0.0f;
        }
    }
    if ((int)threadIdx.x < h)
        freq[threadIdx.x] = fv;
    __syncthreads();
    if constexpr (BWD) {
        // The wave's stages in pairs through a loop with one exit; an odd count
        // ends with one stage past the end (placeholder rows: nothing stored,
        // zero gradient terms).  The two-exit loop below joins at its head a
        // path with the second stage's loads in flight, so the compiler waits
        // there for every load; the backward gains from keeping both stages in
        // flight, the forward (more waves per SIMD) does not.
        const int64_t nblk = gwave < p.token_blocks ? (p.token_blocks - 1 - gwave) / nwaves + 1 : 0;
        const int64_t nstage = nblk * nbatch;
        for (int64_t k = 0; k < nstage; k += 2) {
            advance(sa, sb);
            step(sa);
            advance(sb, sa);
            step(sb);
        }
    } else {
        while (sa.valid) {
            advance(sa, sb);
            step(sa);
            if (!sb.valid)
                break;
            advance(sb, sa);
            step(sb);
        }
    }

    if constexpr (BWD) {
        // Fixed-order reduction of the per-lane dw accumulators: LDS [slot][D],
        // slot = wave * RW + row-in-group, then one thread per channel sums the
        // slots in order into this workgroup's partial.  Partials are stored
        // column-major, [2D][gridDim.x], so the finalize reads each column
        // contiguously.
        const int slot = wave * RW + ln.rho;
        const int64_t P = gridDim.x;
        const int nsets = has_b ? 4 : 2;  // dwq, dwk [, dbq, dbk]
#pragma unroll
        for (int s = 0; s < kAcc; ++s) {
            if (s >= nsets)
                break;
            __syncthreads();
#pragma unroll
            for (int e = 0; e < E; ++e)
                red[slot * D + ln.ch * E + e] = acc[s][e];
            __syncthreads();
            for (int c = threadIdx.x; c < D; c += kThreads) {
                float t = 0.0f;
                for (int k = 0; k < kWaves * RW; ++k)
                    t += red[k * D + c];
                p.partials[(int64_t)(s * D + c) * P + blockIdx.x] = t;
            }
        }
    }
}

// Where column c of the weight and bias gradients goes: columns [0, nq) are
// dwq, [nq, nq + nk) dwk, then nq of dbq and nk of dbk.  Null: not wanted.
struct GradCols {
    void *out[4];  // dwq, dwk, dbq, dbk
    int n[2];      // columns of a q gradient and of a k gradient
    __device__ inline void *locate(int c, int *i) const
    {
        for (int s = 0; s < 4; ++s) {
            const int w = n[s & 1];
            if (c < w) {
                *i = c;
                return out[s];
            }
            c -= w;
        }
        return nullptr;
    }
};

// Column c of the weight (and bias) gradients = sum over the P workgroup
// partials of column c (stored column-major, partials[c * P + b]) in a fixed
// order: one wave per column; lane k adds rows k, k + 64, k + 128, ... (all its
// loads issued first, coalesced across the wave), then a fixed butterfly over
// the 64 lanes; lane 0 stores.  Columns map to outputs as in GradCols; a
// column whose output pointer is null is skipped.
template <typename IO>
__global__ __launch_bounds__(kFinalizeThreads) void qknr_dw_finalize_kernel(
    const float *__restrict__ partials, int P, int cols, GradCols gc)
{
    constexpr int kRowsPerLane = kMaxBwdBlocks / 64;
    const int c = blockIdx.x * (kFinalizeThreads / 64) + (int)(threadIdx.x >> 6);
    const int lane = (int)(threadIdx.x & 63);
    if (c >= cols)
        return;  // c is the same for the whole wave
    int oc = 0;
    void *const out = gc.locate(c, &oc);
    if (!out)
        return;
    const float *col = partials + (int64_t)c * P;
    float v[kRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        const int b = lane + 64 * i;
        v[i] = b < P ? col[b] : 0.0f;
    }
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
        t += v[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        t += __shfl_xor(t, off, 64);
    if (lane == 0)
        Io<IO>::store_scalar(out, oc, t);
}

// ---- norm groups and per-head weights ------------------------------------------
//
// Heads in groups of p.group[0] (q) and p.group[1] (k) share the mean and the
// inverse RMS of their group's values ("QK-Normed MLA: QK normalization without
// full key caching", abstract: one dynamic inverse-RMS scalar per token and head
// group; a group of every head is the layerwise QK-Norm of the SwiftQK
// abstract), and with p.head_w the weights, biases and their gradients are
// [H, D].  RoPE still rotates each head on its own.  The statistics of a group
// need all of its rows, so this kernel gives a workgroup whole tokens: tpi =
// p.tb_tokens tokens per iteration, every 16-byte chunk of them held by one
// of the workgroup's threads (group_threads x group_slots chunks).  A row's C
// chunks sit in C consecutive lanes (C divides 64), so the
// RoPE partner and the
// row sums use the same lane exchanges as qknr_kernel.  Row sums go through
// LDS and each group's sum adds its rows in order: deterministic.
//
// Backward weight/bias gradients: every slot accumulates g xh (and g) of its
// chunk over the workgroup's iterations in registers; at the end the slots go
// to LDS and each gradient column adds the slots that hold it in a fixed order
// (tokens, then rows of its tensor for [D] weights) into the workgroup's
// partial row.  Partials are row-major here, [P][cols].
constexpr int kGroupThreadsFwd = 512;   // 8 waves: one or more whole tokens per iteration
constexpr int kGroupThreadsBwd = 512;   // (two workgroups share a CU)
constexpr int kGroupSlotsFwd = 4;       // chunks per thread: 2048 chunks per iteration
// Backward: x, dy and the dw / db accumulators per slot.  bf16 runs at two
// waves per SIMD whatever its register count below 256, so it takes three
// slots (1536 chunks: two 7B-shaped tokens per iteration instead of one);
// fp32 stays at two (1024 chunks), which keeps it at four waves per SIMD.
constexpr int group_slots(bool bwd, int elems_per_chunk)
{
    return bwd ? (elems_per_chunk == 8 ? 3 : 2) : kGroupSlotsFwd;
}
constexpr int kGroupMaxRows = kGroupThreadsFwd * kGroupSlotsFwd / 8;  // rows per iteration (C >= 8)
constexpr int group_threads(bool bwd) { return bwd ? kGroupThreadsBwd : kGroupThreadsFwd; }
constexpr int kGroupMaxCosSin = 1024;                    // tpi * rotary_dim / 2
// s_waitcnt immediate: vmcnt(0); expcnt and lgkmcnt not waited on
constexpr int kWaitVmcnt0 = 0x0F70;

// Forward: at most 128 VGPRs, so that two 8-wave workgroups share a CU.
// SLOT (forward only): K rows go to the rows a slot map names.
template <typename IO, int D, bool BWD, bool IL, bool SLOT>
__global__ __launch_bounds__(group_threads(BWD)) __attribute__((amdgpu_waves_per_eu(
    BWD ? 2 : 4, 8))) void qknr_group_kernel(const Params p)
{
    using IOT = Io<IO>;
    using S = Shape<IO, D>;
    constexpr int E = S::E, C = S::C, K = group_slots(BWD, S::E);
    constexpr int kGroupThreads = group_threads(BWD);
    __shared__ float rs[kGroupMaxRows];          // row sums [token][row]
    __shared__ float gsum[kGroupMaxRows];        // group means, at the group's first row
    __shared__ float4 cs4[kGroupMaxCosSin / 2 + E / 2];  // [token][i]: (a cos, a sin), then E identities
    float2 *const cs = reinterpret_cast<float2 *>(cs4);
    __shared__ double freq[D / 2];
    __shared__ int32_t posl[kGroupThreads];
    static_assert(!(BWD && SLOT), "slot-mapped output is a forward option");
    __shared__ int64_t slotl[SLOT ? kGroupThreads : 1];  // K output rows (slot map)
    __shared__ float red[BWD ? K * kGroupThreads * E : 1];
    // Weight chunks, then (forward) bias chunks, staged once per workgroup:
    // [wrows][C] each, wrows = hq + hkv heads for [H, D] weights, else 2 (q, k);
    // the host sizes it (group_lds_bytes).
    extern __shared__ u32x4 wlds[];

    const int t = threadIdx.x;
    const Lane<IO, D, IL> ln(t & 63, p.rotary_dim);
    const int h = p.rotary_dim >> 1;
    const int hq = p.heads[0], rpt = p.heads[0] + p.heads[1];
    const int ngq = hq / p.group[0], ngroups = ngq + p.heads[1] / p.group[1];  // groups per token
    const int N = rpt * C;          // chunks per token
    const int tpi = p.tb_tokens;
    const int cols_q = p.head_w ? hq * D : D, cols_k = p.head_w ? p.heads[1] * D : D;
    const int cols = 2 * (cols_q + cols_k);
    const float eps = p.eps;
    // Q / K bases and strides as opaque scalars: a slot picks its tensor with
    // a select.  (Indexed by a per-lane tensor number, the kernel arguments
    // become a vector load and a full memory wait in front of every access.)
    const IO *xq = static_cast<const IO *>(p.x[0]), *xk = static_cast<const IO *>(p.x[1]);
    const IO *gq = static_cast<const IO *>(p.dy[0]), *gk = static_cast<const IO *>(p.dy[1]);
    IO *oq = static_cast<IO *>(p.out[0]), *ok = static_cast<IO *>(p.out[1]);
    int64_t xsq = p.xs[0], xsk = p.xs[1], gsq = p.ds[0], gsk = p.ds[1];
    int64_t osq = p.os[0], osk = p.os[1];
    asm volatile("" : "+s"(xq), "+s"(xk), "+s"(gq), "+s"(gk), "+s"(oq), "+s"(ok));
    asm volatile("" : "+s"(xsq), "+s"(xsk), "+s"(gsq), "+s"(gsk), "+s"(osq), "+s"(osk));
    for (int i = t; i < h; i += kGroupThreads)
        freq[i] = p.inv_freq[i];
    const int wrows = p.head_w ? rpt : 2;
    const int nw = p.has_w ? wrows * C : 0, nwb = nw + (!BWD && p.has_b ? wrows * C : 0);
    for (int i = t; i < nwb; i += kGroupThreads) {
        const bool isb = i >= nw;
        const int j = isb ? i - nw : i, wr = j / C, c = j - wr * C;
        const int seg = p.head_w ? (wr >= hq ? 1 : 0) : wr;
        const int head = p.head_w ? (seg ? wr - hq : wr) : 0;
        const void *src = isb ? p.b[seg] : p.w[seg];
        wlds[i] = ld16_cached(static_cast<const IO *>(src) + head * D + c * E);
    }
    float2 *const cs_id = cs + kGroupMaxCosSin;   // (1, 0) entries for unrotated chunks
    if (t < E)
        cs_id[t] = make_float2(1.0f, 0.0f);
    // This lane's run of table entries for a row of token tl starts at
    // cs_lane0 + tl * cs_tok: E entries (half-split: pairs pc E ...) or E / 2
    // (interleaved: pairs ch E / 2 ..., each used by two elements).
    const int cs_off = ln.rot ? (IL ? ln.ch * E / 2 : ln.pc * E) : 0;
    const int cs_tok = ln.rot ? h : 0;
    const float ssign = (IL || !ln.first) ? 1.0f : -1.0f;

    // Fixed per slot k (chunk t + kGroupThreads k of an iteration): token in the
    // iteration and row (q heads, then k heads), or -1; first row and size of
    // the row's norm group.
    int code[K], grp[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int idx = t + kGroupThreads * k;
        const int tl = idx / N, row = (idx - tl * N) / C;
        const bool on = tl < tpi;
        const bool seg = row >= hq;
        const int gs = seg ? p.group[1] : p.group[0];
        const int g0 = seg ? hq + ((row - hq) / gs) * gs : (row / gs) * gs;
        code[k] = on ? (tl << 16) | row : -1;
        grp[k] = (g0 << 12) | gs;
    }
    // per slot: sum of g xh (dw) and of g (db) of its chunk
    float accw[BWD ? K : 1][E], accb[BWD ? K : 1][E];
    if constexpr (BWD) {
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                accw[k][e] = accb[k][e] = 0.0f;
    }
    const bool layernorm = p.layernorm != 0;
    const int64_t iters = (p.tokens + tpi - 1) / tpi;

    // The chunks (and positions) of one iteration.  (A second set prefetching
    // the next iteration measured slower in the forward, which runs two
    // workgroups per CU; the bf16 backward prefetches, below.)
    struct Chunks {
        u32x4 x[K];
        u32x4 dy[BWD ? K : 1];
        int32_t pos;
        int64_t slot;  // forward with a slot map: K output row of token t (t < tpi)
    };
    constexpr bool slots = SLOT;
    auto load = [&](Chunks &c, int64_t it) {
        // Recompute the per-slot addresses in every iteration instead of
        // keeping them (hoisted out of the loop, they outgrow the registers):
        // the empty asm makes the slot codes opaque to that hoisting.
#pragma unroll
        for (int k = 0; k < K; ++k)
            asm volatile("" : "+v"(code[k]), "+v"(grp[k]));
        const bool on = it < iters;
        const int64_t tok0 = it * tpi;
        c.pos = on && t < tpi && tok0 + t < p.tokens ? p.pos[tok0 + t] : 0;
        if constexpr (SLOT) {
            c.slot = on && t < tpi && tok0 + t < p.tokens ? p.slots[tok0 + t] : -1;
            if (c.slot >= p.k_out_rows)
                c.slot = -1;  // outside k_out: skipped like a negative slot
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int tl = code[k] >> 16, row = code[k] & 0xffff;
            const bool isk = row >= hq;
            const int head = isk ? row - hq : row;
            const int64_t tok = tok0 + tl;
            c.x[k] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (BWD)
                c.dy[k] = u32x4{0u, 0u, 0u, 0u};
            if (on && code[k] >= 0 && tok < p.tokens) {
                c.x[k] = ld16((isk ? xk : xq) + tok * (isk ? xsk : xsq) + head * D + ln.ch * E);
                if constexpr (BWD)
                    c.dy[k] = ld16((isk ? gk : gq) + tok * (isk ? gsk : gsq) + head * D + ln.ch * E);
            }
        }
    };
    auto process = [&](const Chunks &ch, int64_t it) {
        const int64_t tok0 = it * tpi;
        const u32x4 *const xv = ch.x;
        const u32x4 *const dv = ch.dy;
        if (t < tpi) {
            posl[t] = ch.pos;
            if constexpr (SLOT)
                slotl[t] = ch.slot;
        }
        __syncthreads();  // positions visible; previous iteration's LDS reads done
        for (int v = t; v < tpi * h; v += kGroupThreads) {
            const int tl = v / h;
            cs[v] = cos_sin_f32((double)posl[tl] * freq[v - tl * h], p.attn);
        }

        // Group statistics: the row sums of each slot into LDS; then one
        // wave per (token, group): lane l adds rows l, l + 64, ... of the
        // group in order, a fixed butterfly adds the 64 lanes, and the sum is
        // divided by the group's size; then every slot reads its group's.
        // (The next call writes rs only after its own first barrier, which
        // every thread reaches after reading gsum here, and gsum only after
        // its second: no trailing barrier is needed.)
        auto group_stat = [&](const float *part, float *res) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const float v = group_sum<C>(part[k]);
                if (code[k] >= 0 && (t % C) == 0)
                    rs[(code[k] >> 16) * rpt + (code[k] & 0xffff)] = v;
            }
            __syncthreads();
            for (int j = t >> 6; j < tpi * ngroups; j += kGroupThreads / 64) {
                const int tl = j / ngroups, gi = j - tl * ngroups;
                const bool isk = gi >= ngq;
                const int gs = isk ? p.group[1] : p.group[0];
                const int base = tl * rpt + (isk ? hq + (gi - ngq) * gs : gi * gs);
                float v = 0.0f;
                for (int r = t & 63; r < gs; r += 64)
                    v += rs[base + r];
                v = group_sum<64>(v);
                if ((t & 63) == 0)
                    gsum[base] = v / (float)(gs * D);
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < K; ++k)
                res[k] = gsum[(code[k] >= 0 ? (code[k] >> 16) : 0) * rpt + (grp[k] >> 12)];
        };
        float mk[K], rk[K], part[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            mk[k] = 0.0f;
        if (layernorm) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float x[E];
                IOT::unpack(xv[k], x);
                float v = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v += x[e];
                part[k] = v;
            }
            group_stat(part, mk);
        }
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float x[E];
            IOT::unpack(xv[k], x);
            float v = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = x[e] - mk[k];
                v = fmaf(d, d, v);
            }
            part[k] = v;
        }
        group_stat(part, rk);
#pragma unroll
        for (int k = 0; k < K; ++k)
            rk[k] = rsqrtf(rk[k] + eps);

        // per-slot helpers
        // LDS chunk of this slot's weight (bias: + nw)
        auto wchunk = [&](int k) {
            const int row = code[k] >= 0 ? code[k] & 0xffff : 0;
            return (p.head_w ? row : (row >= hq ? 1 : 0)) * C + ln.ch;
        };
        auto weights = [&](int k, float *w) {
            if (p.has_w) {
                IOT::unpack(wlds[wchunk(k)], w);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    w[e] = 1.0f;
            }
        };
        // c and signed s of each element: half-split pairs (i, i+h) sit in
        // mirrored lanes, y = n c - n' s in the first half, + n' s in the
        // second; interleaved pairs (2i, 2i+1): - at even elements, + at odd.
        auto cos_sin = [&](int k, float *c, float *sn) {
            const int tl = code[k] >= 0 ? code[k] >> 16 : 0;
            const float4 *src = reinterpret_cast<const float4 *>(
                (ln.rot ? cs + cs_off : cs_id) + tl * cs_tok);
            if constexpr (IL) {
#pragma unroll
                for (int e = 0; e < E / 4; ++e) {
                    const float4 v = src[e];   // pairs 2e, 2e + 1 of the chunk
                    c[4 * e] = c[4 * e + 1] = v.x;
                    c[4 * e + 2] = c[4 * e + 3] = v.z;
                    sn[4 * e] = -v.y;
                    sn[4 * e + 1] = v.y;
                    sn[4 * e + 2] = -v.w;
                    sn[4 * e + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < E / 2; ++e) {
                    const float4 v = src[e];
                    c[2 * e] = v.x;
                    sn[2 * e] = ssign * v.y;
                    c[2 * e + 1] = v.z;
                    sn[2 * e + 1] = ssign * v.w;
                }
            }
        };
        // output row: the token, or for K rows with a slot map the token's slot
        // (negative: not stored)
        auto out_row = [&](int k) {
            const int tl = code[k] >= 0 ? code[k] >> 16 : 0;  // unused slots: any valid entry
            return slots && (code[k] & 0xffff) >= hq ? slotl[tl] : tok0 + tl;
        };
        auto out_ptr = [&](int k) {
            const int row = code[k] & 0xffff;
            const bool isk = row >= hq;
            const int head = isk ? row - hq : row;
            return (isk ? ok : oq) + out_row(k) * (isk ? osk : osq) + head * D + ln.ch * E;
        };
        auto live = [&](int k) {
            return code[k] >= 0 && tok0 + (code[k] >> 16) < p.tokens && out_row(k) >= 0;
        };

        if constexpr (!BWD) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float x[E], w[E], n[E], y[E], c[E], sn[E];
                IOT::unpack(xv[k], x);
                weights(k, w);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    n[e] = (x[e] - mk[k]) * rk[k] * w[e];
                if (p.has_b) {
                    float b[E];
                    IOT::unpack(wlds[nw + wchunk(k)], b);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        n[e] += b[e];
                }
                cos_sin(k, c, sn);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    y[e] = fmaf(n[e], c[e], (IL ? n[e ^ 1] : mirror<C>(n[e])) * sn[e]);
                if (live(k))
                    st16(out_ptr(k), IOT::pack(y));
            }
        } else {
            // g = R^T dy (rotation by -phi), recomputed where used
            auto grad_in = [&](int k, float *g) {
                float c[E], sn[E], gp[E];
                IOT::unpack(dv[k], g);
                if constexpr (IL) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        gp[e] = g[e ^ 1];
                } else {
                    u32x4 dyp;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dyp[i] = mirror<C>(dv[k][i]);
                    IOT::unpack(dyp, gp);
                }
                cos_sin(k, c, sn);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    g[e] = fmaf(g[e], c[e], -gp[e] * sn[e]);
            };
            // bf16: g, xh and u = w g of the first pass stay in registers for
            // the second (at this kernel's occupancy the registers are free);
            // fp32 recomputes them, keeping four waves per SIMD.
            constexpr bool kKeep = E == 8;
            constexpr int KK = kKeep ? K : 1;
            float kg[KK][E], kxh[KK][E], ku[KK][E];
            float pd[K], su[K], mean[K], mu[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float x[E], w[E], g[E];
                IOT::unpack(xv[k], x);
                weights(k, w);
                grad_in(k, g);
                float a = 0.0f, b2 = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float xh = (x[e] - mk[k]) * rk[k];
                    const float u = w[e] * g[e];
                    a = fmaf(u, xh, a);
                    b2 += u;
                    if constexpr (kKeep) {
                        kg[k][e] = g[e];
                        kxh[k][e] = xh;
                        ku[k][e] = u;
                    }
                }
                pd[k] = a;
                su[k] = b2;
            }
            group_stat(pd, mean);
            if (layernorm)
                group_stat(su, mu);
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float g[E], xh[E], u[E], dx[E];
                if constexpr (kKeep) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        g[e] = kg[k][e];
                        xh[e] = kxh[k][e];
                        u[e] = ku[k][e];
                    }
                } else {
                    float x[E], w[E];
                    IOT::unpack(xv[k], x);
                    weights(k, w);
                    grad_in(k, g);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        xh[e] = (x[e] - mk[k]) * rk[k];
                        u[e] = w[e] * g[e];
                    }
                }
                const float m2 = layernorm ? mu[k] : 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    dx[e] = rk[k] * fmaf(-xh[e], mean[k], u[e] - m2);
                if (!live(k))
                    continue;
                st16(out_ptr(k), IOT::pack(dx));
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    accw[k][e] = fmaf(g[e], xh[e], accw[k][e]);
                    accb[k][e] += g[e];
                }
            }
        }
        };

    if constexpr (BWD && E == 8) {
        // bf16 backward: one workgroup per CU, so nothing else hides an
        // iteration's load latency; the next iteration's chunks are loaded
        // while this one is processed.  The explicit wait at the loop head
        // covers this iteration's chunks (and earlier stores) before the next
        // loads are issued; without it the compiler's wait for this
        // iteration's data, with stores outstanding, would be a full drain
        // that includes the prefetch.
        Chunks cur;
        load(cur, blockIdx.x);
        for (int64_t it = blockIdx.x; it < iters; it += gridDim.x) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            Chunks nxt;
            load(nxt, it + gridDim.x);
            process(cur, it);
            cur = nxt;
        }
    } else {
        for (int64_t it = blockIdx.x; it < iters; it += gridDim.x) {
            Chunks c;
            load(c, it);
            process(c, it);
        }
    }

    if constexpr (BWD) {
        // Slot (k, t) holds chunk idx = t + kGroupThreads k of an iteration, i.e.
        // token idx / N, row (idx % N) / C, lane position idx % C.  Column j of
        // a row is element j % E of the chunk in the lane position i0 holding
        // chunk j / E.
        float *prow = p.partials + (int64_t)blockIdx.x * cols;
        const int half = cols / 2;   // dw columns, then as many db columns
        for (int pass = 0; pass < (p.has_b ? 2 : 1); ++pass) {
            __syncthreads();
#pragma unroll
            for (int k = 0; k < K; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    red[(k * kGroupThreads + t) * E + e] = pass ? accb[k][e] : accw[k][e];
            __syncthreads();
            for (int c = t; c < half; c += kGroupThreads) {
                int row0, nrows, j;
                if (p.head_w) {
                    row0 = c / D;               // one row (head) per column
                    nrows = 1;
                    j = c - row0 * D;
                } else {
                    const int seg = c / D;      // every row of the column's tensor
                    row0 = seg ? hq : 0;
                    nrows = seg ? rpt - hq : hq;
                    j = c - seg * D;
                }
                int i0 = 0;
                for (int i = 0; i < C; ++i)
                    if (Lane<IO, D, IL>(i, p.rotary_dim).ch == j / E)
                        i0 = i;
                float v = 0.0f;
                for (int tl = 0; tl < tpi; ++tl)
                    for (int r = row0; r < row0 + nrows; ++r)
                        v += red[((tl * N + r * C + i0) * E) + j % E];
                prow[pass * half + c] = v;
            }
        }
    }
}

// Row-major partials [P][cols] (P <= kMaxBwdBlocks) of the norm-group
// kernels: a workgroup sums 16 consecutive columns (a 64-byte slice of each
// partial row), so the launch spreads over many CUs.  Its 1024 threads are 64
// row lanes of 16 columns; row lane l adds rows l, l + 64, l + 128, ... (all
// its loads issued first) in order, then thread c < 16 adds the 64 row lanes'
// sums in order and stores column c.  Columns whose output is null are neither
// read nor stored.
constexpr int kGroupFinalizeCols = 16;
constexpr int kGroupFinalizeThreads = 1024;

template <typename IO>
__global__ __launch_bounds__(kGroupFinalizeThreads) void qknr_group_finalize_kernel(
    const float *__restrict__ partials, int P, int cols, GradCols gc)
{
    constexpr int W = kGroupFinalizeCols, L = kGroupFinalizeThreads / W;
    constexpr int kRowsPerLane = kMaxBwdBlocks / L;
    static_assert(kMaxBwdBlocks % L == 0, "partial rows split evenly over the row lanes");
    __shared__ float part[L][W];
    const int rl = (int)threadIdx.x / W, cl = (int)threadIdx.x % W;
    const int c = blockIdx.x * W + cl;
    int oc = 0;
    void *const out = c < cols ? gc.locate(c, &oc) : nullptr;
    float v[kRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
        const int b = rl + L * i;
        v[i] = out && b < P ? partials[(int64_t)b * cols + c] : 0.0f;
    }
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
        t += v[i];
    part[rl][cl] = t;
    __syncthreads();
    if (rl == 0 && out) {
        float s = 0.0f;
#pragma unroll
        for (int l = 0; l < L; ++l)
            s += part[l][cl];
        Io<IO>::store_scalar(out, oc, s);
    }
}

// ---- Norm groups within one wave ------------------------------------------------
//
// The same operation as qknr_group_kernel (norm groups, [H, D] weights and
// biases) when every norm group lies within one pipeline stage of two wave
// instructions of rows.  Either a stage holds whole tokens (p.stages = 1: token
// blocks of at most two instructions of rows, e.g. the 16 bf16 rows of 64 of a
// 14 + 2 head token), or a token spans p.stages stages and every group lies in
// one of them (e.g. the 40 rows of a 32 + 8 head token of 128 in five 8-row
// stages, q in groups of 4 heads, k of 8); then wave w always takes stage
// w mod p.stages of its tokens.  Either way a group's statistics need no
// workgroup: each row's sum goes to a wave-private LDS array and the group's
// rows are added in order there.  Everything else is qknr_kernel's: persistent
// waves walk token blocks two stages deep, cos/sin per block in the wave's
// table, chunks in mirrored lanes.  A lane always holds the same (token row,
// chunk) of a block, so the backward accumulates dw (and db) per stage slot
// and reduces them through LDS in a fixed order into row-major partials
// [P][cols] for qknr_group_finalize_kernel.
// At most 3 (forward) and 2 (backward) waves per SIMD: the register budget
// of 168 and 256 VGPRs holds both stages without spilling.
constexpr int kGwMaxWeights = 1024;   // a stage's weights (and biases) as fp32: 2 RW D <= 1024
constexpr int kGwMaxRows = 16;        // rows of a stage: 2 * RW <= 16
constexpr int kGwMaxStages = 32;      // stages per token
constexpr int64_t kSplitTokens = 1024; // forwards of at most this many tokens split tokens over waves

template <typename IO, int D, bool BWD, bool IL, bool SLOT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    BWD ? 2 : 3, 8))) void qknr_gwave_kernel(const Params p)
{
    static_assert(!(BWD && SLOT), "slot-mapped output is a forward option");
    using IOT = Io<IO>;
    using S = Shape<IO, D>;
    constexpr int E = S::E, C = S::C, RW = S::RW, U = 2;
    static_assert(U * RW <= kGwMaxRows, "rows of a stage");
    constexpr int kCsStride = D / 2;
    constexpr int kCsWave = 2 * S::kCsCap + E;
    __shared__ float4 cs_store[kWaves * kCsWave / 2];
    static_assert(U * RW * D <= kGwMaxWeights, "a stage's weights");
    __shared__ float wls[kWaves][U * RW * D];          // weights of each wave's stage rows
    __shared__ float bls[BWD ? 1 : kWaves][BWD ? 1 : U * RW * D];  // biases (forward)
    __shared__ float4 rsum[kWaves][kGwMaxRows / 4];  // row sums of the wave's stage
    __shared__ float gstat[kWaves][kGwMaxRows];               // their groups' statistics
    constexpr int kRedSlots = kWaves * U * 64 * E;       // one gradient set's slots
    __shared__ float red[BWD ? 2 * kRedSlots : 1];       // dw slots, then db slots
    __shared__ double freq[D / 2];
    touch_params(p);

    // the wave index as a scalar, so the stage and block bookkeeping below
    // stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    float2 *cs = reinterpret_cast<float2 *>(cs_store) + wave * kCsWave;
    float2 *cs_id = cs + 2 * S::kCsCap;
    const Lane<IO, D, IL> ln(lane, p.rotary_dim);
    const int h = p.rotary_dim >> 1;
    const int nvals = p.tb_tokens * h;
    if (lane < E)
        cs_id[lane] = make_float2(1.0f, 0.0f);
    const float2 *cs_row0 = IL ? cs + ln.ch * E : (ln.first ? cs : cs + S::kCsCap) + ln.pc * E;
    const float4 *cs_lane = reinterpret_cast<const float4 *>(ln.rot ? cs_row0 : cs_id);
    const int cs_tok = ln.rot ? (IL ? D / 2 : kCsStride / 2) : 0;

    const int hq = p.heads[0], rpt = p.rows_per_token;
    const bool head_w = p.head_w != 0;
    const int rows_w = head_w ? rpt : 2;
    // This wave's stage of a token block: rows srow .. srow + U RW - 1 of the
    // block (token-major); with one stage per block it is the whole block.
    const int nst = p.stages;
    const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
    const int sidx = (int)(gw % nst);
    const int srow = sidx * U * RW;
    // The weights (and biases) of the stage's rows, row j at j D, 16-byte
    // chunks per lane from base pointers held as scalars (a per-lane index
    // into the argument arrays would load the pointer per lane); rows past
    // the block's tokens get 1 (and 0) and are never stored.
    float *const wl = wls[wave];
    // Loaded into registers here and written to LDS after the first stage's
    // loads are issued (below), with no branch around the loads: rows with no
    // weight (bias) to read take q's first 16 bytes, replaced when written.
    constexpr int kWc = U * RW * C / 64;   // weight chunks per lane
    static_assert(U * RW * C % 64 == 0, "whole chunks per lane");
    u32x4 wraw[kWc], braw[kWc];
    bool wreal[kWc], breal[kWc];
    {
        const IO *const w0 = static_cast<const IO *>(p.w[0]), *const w1 = static_cast<const IO *>(p.w[1]);
        const IO *const b0 = static_cast<const IO *>(p.b[0]), *const b1 = static_cast<const IO *>(p.b[1]);
#pragma unroll
        for (int k = 0; k < kWc; ++k) {
            const int c = lane + 64 * k;
            const int j = c / C, qc = c - j * C, row = srow + j, tl = row / rpt;
            const int in_tok = row - tl * rpt, seg = in_tok >= hq ? 1 : 0;
            const int64_t off = (head_w ? (int64_t)(seg ? in_tok - hq : in_tok) * D : 0) + qc * E;
            const bool real = tl < p.tb_tokens;
            wreal[k] = p.has_w && real;
            wraw[k] = ld16_cached(wreal[k] ? (const void *)((seg ? w1 : w0) + off) : p.x[0]);
            if constexpr (!BWD) {
                breal[k] = p.has_b && real;
                braw[k] = ld16_cached(breal[k] ? (const void *)((seg ? b1 : b0) + off) : p.x[0]);
            }
        }
    }
    static_assert(D / 2 <= kThreads, "one frequency per thread");
    const double fv = (int)threadIdx.x < h ? p.inv_freq[threadIdx.x] : 0.0;
    // the staged values to LDS: the stage's weight rows at j D (1 where there
    // is none), biases likewise (0), the frequencies
    auto to_lds = [&]() {
#pragma unroll
        for (int k = 0; k < kWc; ++k) {
            const int c = lane + 64 * k, j = c / C, qc = c - j * C;
            float v[E];
            IOT::unpack(wraw[k], v);
#pragma unroll
            for (int e = 0; e < E; ++e)
                wl[j * D + qc * E + e] = wreal[k] ? v[e] : 1.0f;
            if constexpr (!BWD) {
                IOT::unpack(braw[k], v);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    bls[wave][j * D + qc * E + e] = breal[k] ? v[e] : 0.0f;
            }
        }
        if ((int)threadIdx.x < h)
            freq[threadIdx.x] = fv;
        __syncthreads();
    };
    // the backward (at its register limit) writes them before the rest of
    // its set-up; the forward after its first stage's loads are issued
    if constexpr (BWD)
        to_lds();

    int vcode[S::kValsPerLane];
    cos_sin_codes<IO, D>(h, nvals, vcode);

    // Fixed per slot u: its row within the stage.
    int rr[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        rr[u] = u * RW + ln.rho;
    // Lane j < U RW stands for row j of the stage: the stage rows of its norm
    // group (first, count; the group lies within the stage) and 1 / (count D).
    // Rows past the block's tokens (never stored) have no group and a
    // statistic of 0.
    int gbase = 0, gsz = 0;
    float ginv = 0.0f;
    if (lane < U * RW) {
        const int row = srow + lane, tl = row / rpt, in_tok = row - tl * rpt;
        const bool isk = in_tok >= hq;
        const int gs = isk ? p.group[1] : p.group[0];
        gbase = tl * rpt + (isk ? hq + ((in_tok - hq) / gs) * gs : (in_tok / gs) * gs) - srow;
        gsz = tl < p.tb_tokens ? gs : 0;
        ginv = gsz ? 1.0f / (float)(gsz * D) : 0.0f;
    }
    float accw[BWD ? U : 1][E], accb[BWD ? U : 1][E];
    if constexpr (BWD) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                accw[u][e] = accb[u][e] = 0.0f;
    }
    const bool layernorm = p.layernorm != 0;
    const bool has_b = p.has_b != 0;
    // every row of the stage belongs to a token of its block
    const bool rows_full = srow + U * RW <= p.tb_tokens * rpt;
    // the waves of this stage, and this wave's place among them (the grid
    // holds a multiple of nst waves)
    const int64_t gwave = gw / nst;
    const int64_t nwaves = (int64_t)gridDim.x * kWaves / nst;
    const float eps = p.eps;
    IO *const out0 = static_cast<IO *>(p.out[0]);
    IO *const out1 = static_cast<IO *>(p.out[1]);
    const int64_t os0 = p.os[0], os1 = p.os[1];
    float *const rs = reinterpret_cast<float *>(rsum[wave]);
    float *const gst = gstat[wave];

    // The statistic of each slot's norm group: the row sums go to the wave's
    // LDS array; lane j reads them back whole (vector reads), adds row j's
    // group in order (the other rows add +0, which changes no sum that starts
    // at +0) and scales it; every lane then reads its rows' results.
    auto group_stat = [&](const float *part, float *res) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float v = group_sum<C>(part[u]);
            if ((lane % C) == 0)
                rs[rr[u]] = v;
        }
        wave_sync();
        float a[U * RW];
        if constexpr (U * RW % 4 == 0) {
#pragma unroll
            for (int q = 0; q < U * RW / 4; ++q) {
                const float4 t = rsum[wave][q];
                a[4 * q] = t.x; a[4 * q + 1] = t.y; a[4 * q + 2] = t.z; a[4 * q + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < U * RW; ++j)
                a[j] = rs[j];
        }
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < U * RW; ++j)
            v += (unsigned)(j - gbase) < (unsigned)gsz ? a[j] : 0.0f;
        if (lane < U * RW)
            gst[lane] = v * ginv;
        wave_sync();
#pragma unroll
        for (int u = 0; u < U; ++u)
            res[u] = gst[rr[u]];
    };

    auto step = [&](Stage<IO, D, U, BWD> &st) {
        wave_sync();  // previous block's table reads are done
        fill_cos_sin<IO, D, IL>(st.pos, freq, p.attn, vcode, nvals, cs);
        wave_sync();
        float x[U][E], r[U], part[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            IOT::unpack(st.x[u], x[u]);
        if (layernorm) {
            // x - mean of the group, in place
            float m[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float v = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v += x[u][e];
                part[u] = v;
            }
            group_stat(part, m);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    x[u][e] -= m[u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                v = fmaf(x[u][e], x[u][e], v);
            part[u] = v;
        }
        group_stat(part, r);
#pragma unroll
        for (int u = 0; u < U; ++u)
            r[u] = rsqrtf(r[u] + eps);

        // the lane's cos/sin and weights of slot u's row
        auto csw = [&](int u, float *c, float *sn, float *w) {
            const float4 *src = cs_lane + st.r[u].tl * cs_tok;
#pragma unroll
            for (int e = 0; e < E / 2; ++e) {
                const float4 v = src[e];
                c[2 * e] = v.x;
                sn[2 * e] = v.y;
                c[2 * e + 1] = v.z;
                sn[2 * e + 1] = v.w;
            }
            const float4 *ws = reinterpret_cast<const float4 *>(wl + rr[u] * D + ln.ch * E);
#pragma unroll
            for (int e = 0; e < E / 4; ++e) {
                const float4 a = ws[e];
                w[4 * e] = a.x; w[4 * e + 1] = a.y; w[4 * e + 2] = a.z; w[4 * e + 3] = a.w;
            }
        };
        auto out_ptr = [&](int u, bool &store) {
            const RowRef &rf = st.r[u];
            store = rf.valid;
            int64_t orow = rf.tok;
            if constexpr (SLOT) {
                const int src = rf.tl << 2;
                const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(
                    src, (int)(uint32_t)(uint64_t)st.slot);
                const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(
                    src, (int)(uint32_t)((uint64_t)st.slot >> 32));
                const int64_t sl = (int64_t)(((uint64_t)hi << 32) | lo);
                if (rf.seg) {
                    orow = sl;
                    store = store && sl >= 0;
                }
            }
            return (rf.seg ? out1 : out0) + (orow * (rf.seg ? os1 : os0) + rf.hofs);
        };
        if constexpr (!BWD) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float n[E], y[E], c[E], sn[E], w[E];
                csw(u, c, sn, w);
                const float4 *bs = reinterpret_cast<const float4 *>(bls[wave] + rr[u] * D + ln.ch * E);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    n[e] = x[u][e] * r[u] * w[e];
                if (has_b) {
#pragma unroll
                    for (int e = 0; e < E / 4; ++e) {
                        const float4 a = bs[e];
                        n[4 * e] += a.x; n[4 * e + 1] += a.y; n[4 * e + 2] += a.z; n[4 * e + 3] += a.w;
                    }
                }
#pragma unroll
                for (int e = 0; e < E; ++e)
                    y[e] = fmaf(n[e], c[e], (IL ? n[e ^ 1] : mirror<C>(n[e])) * sn[e]);
                const u32x4 packed = IOT::pack(y);
                bool store;
                IO *o = out_ptr(u, store);
                if (store)
                    st16(o, packed);
            }
        } else {
            float g[U][E], xh[U][E], uu[U][E], pd[U], mean[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float gp[E], c[E], sn[E], w[E];
                csw(u, c, sn, w);
                IOT::unpack(st.dy[u], g[u]);
                if constexpr (IL) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        gp[e] = g[u][e ^ 1];
                } else {
                    u32x4 dyp;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dyp[i] = mirror<C>(st.dy[u][i]);
                    IOT::unpack(dyp, gp);
                }
                float a = 0.0f;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    g[u][e] = fmaf(g[u][e], c[e], -gp[e] * sn[e]);
                    xh[u][e] = x[u][e] * r[u];
                    uu[u][e] = w[e] * g[u][e];
                    a = fmaf(uu[u][e], xh[u][e], a);
                }
                pd[u] = a;
            }
            group_stat(pd, mean);
            if (layernorm) {
                // u - its group mean, in place
                float su[U], mu[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    float b2 = 0.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        b2 += uu[u][e];
                    su[u] = b2;
                }
                group_stat(su, mu);
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        uu[u][e] -= mu[u];
            }
            // rows past the end (placeholder data) add exact zeros
            if (!(rows_full && (st.tb + 1) * p.tb_tokens <= p.tokens)) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float mv = st.r[u].valid ? 1.0f : 0.0f;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        g[u][e] *= mv;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dx[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    dx[e] = r[u] * fmaf(-xh[u][e], mean[u], uu[u][e]);
                const u32x4 packed = IOT::pack(dx);
                bool store;
                IO *o = out_ptr(u, store);
                mem_priority<true>(true);
                if (store)
                    st16(o, packed);
                mem_priority<true>(false);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    accw[u][e] = fmaf(g[u][e], xh[u][e], accw[u][e]);
                    accb[u][e] += g[u][e];
                }
            }
        }
    };
    // this lane's rows of a block, the same in every block (token-major: a
    // token's Hq Q rows, then its Hkv K rows); the token count is checked per
    // block
    RowRef fixed[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int row = srow + rr[u], tl = row / rpt, in_tok = row - tl * rpt;
        const int seg = in_tok >= hq ? 1 : 0;
        fixed[u].tok = 0;
        fixed[u].tl = tl;
        fixed[u].seg = seg;
        fixed[u].hofs = (seg ? in_tok - hq : in_tok) * D + ln.ch * E;
        fixed[u].valid = sidx * U + u < p.groups && tl < p.tb_tokens;
    }
    auto advance = [&](const Stage<IO, D, U, BWD> &from, Stage<IO, D, U, BWD> &to) {
        to.batch = sidx;
        to.tb = from.tb + nwaves;
        to.valid = to.tb < p.token_blocks;
        mem_priority<true>(true);
        issue_fixed<IO, D, U, BWD, SLOT>(p, to, fixed);
        mem_priority<true>(false);
    };
    Stage<IO, D, U, BWD> sa, sb;
    sa.tb = gwave;
    sa.batch = sidx;
    sa.valid = sa.tb < p.token_blocks;
    issue_fixed<IO, D, U, BWD, SLOT>(p, sa, fixed);
    if constexpr (!BWD)
        to_lds();
    // The wave's blocks in pairs.  The two-exit loop (a break between the two
    // halves) joins at its head a path with the second block's loads still in
    // flight, so the wait analysis holds every block there until all loads
    // land.  The backward walks the pairs through a loop with one exit
    // instead; an odd count ends with one block past the end, whose rows are
    // placeholders: nothing stored, zero gradient terms.  It holds about 24
    // more VGPRs: the bf16 interleaved D = 64 backward would spill at 256,
    // and the forwards gain nothing, so they keep the two-exit loop.
    constexpr bool kOneExit = BWD && !(IL && D == 64 && sizeof(IO) == 2);
    if constexpr (kOneExit) {
        const int64_t nblk = gwave < p.token_blocks ? (p.token_blocks - 1 - gwave) / nwaves + 1 : 0;
        for (int64_t k = 0; k < nblk; k += 2) {
            advance(sa, sb);
            step(sa);
            advance(sb, sa);
            step(sb);
        }
    } else {
        while (sa.valid) {
            advance(sa, sb);
            step(sa);
            if (!sb.valid)
                break;
            advance(sb, sa);
            step(sb);
        }
    }

    if constexpr (BWD) {
        // Slot (wave, u, lane) holds stage row u RW + rho of every block the
        // wave visited, chunk ch; each gradient column adds, in a fixed order
        // (wave, then token of the block, or stage row for [D] weights), the
        // slots whose row has its weight row and whose lane holds its chunk.
        const int half = rows_w * D;   // dw columns, then as many db columns
        const int cols = 2 * half;
        float *prow = p.partials + (int64_t)blockIdx.x * cols;
        int srw[kWaves];  // first stage row of each wave of the workgroup
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv)
            srw[wv] = (int)(((int64_t)blockIdx.x * kWaves + wv) % nst) * U * RW;
        // Both sets in one pass (red is not used before this point, so one
        // barrier orders the writes before the reads).
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                red[((wave * U + u) * 64 + lane) * E + e] = accw[u][e];
                if (has_b)
                    red[kRedSlots + ((wave * U + u) * 64 + lane) * E + e] = accb[u][e];
            }
        __syncthreads();
        // the lane position within a row that holds chunk jc (inverse of
        // Lane::ch): half-split first halves in place, second halves mirrored,
        // unrotated chunks after the first halves; interleaved in place
        const int hc = (p.rotary_dim / 2) / E;
        for (int cc = threadIdx.x; cc < half; cc += kThreads) {
            const int wr = cc / D, j = cc - wr * D, jc = j / E;
            const int i0 = IL ? jc : (jc < hc ? jc : (jc < 2 * hc ? C - 1 + hc - jc : jc - hc));
            auto slot = [&](int wv, int r) {
                return ((wv * U + r / RW) * 64 + (r % RW) * C + i0) * E + j % E;
            };
            float vw = 0.0f, vb = 0.0f;
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) {
                const int sr = srw[wv];
                if (head_w) {
                    // weight row wr is token row wr of each of the block's tokens
                    for (int tl = 0; tl < p.tb_tokens; ++tl) {
                        const int r = tl * rpt + wr - sr;
                        if (r >= 0 && r < U * RW) {
                            vw += red[slot(wv, r)];
                            vb += has_b ? red[kRedSlots + slot(wv, r)] : 0.0f;
                        }
                    }
                } else {
                    // weight row 0 (q) or 1 (k): every row of that tensor
                    for (int r = 0; r < U * RW; ++r) {
                        const int row = sr + r, tl = row / rpt, in_tok = row - tl * rpt;
                        if (tl < p.tb_tokens && (in_tok >= hq ? 1 : 0) == wr) {
                            vw += red[slot(wv, r)];
                            vb += has_b ? red[kRedSlots + slot(wv, r)] : 0.0f;
                        }
                    }
                }
            }
            prow[cc] = vw;
            if (has_b)
                prow[half + cc] = vb;
        }
    }
}

// ---- Best-Fit-Decreasing packing of documents into buffers ---------------------
//
// The data step in front of the path: documents are packed into buffers of
// `capacity` tokens with Best-Fit Decreasing ("Chronicals", abstract,
// contribution (4)), and the position ids restart at 0 at every document (and
// at the filler that completes a bin), which is what the kernels above take.
// Tie-breaks: longest first, equal lengths in input order; each document into
// the open bin with the least room that fits it (lowest index among equals),
// else a new bin; bins in opening order, documents in placement order, one
// filler segment per bin that is not full.
//
// qknr_bfd_place_kernel (one workgroup): validates the lengths, sorts the
// documents by the 64-bit key (capacity - length) << 32 | index with a bitonic
// sort (ascending key = longest first, stable), then places them in order,
// each document at the minimum of (room << 12 | bin) over the open bins that
// fit it (least room, lowest index among equals): with at most 64 bins one
// wave holds them in registers (a bin per lane); with more, the whole
// workgroup does (1, 2 or 4 bins per thread), a wave minimum and then a
// minimum over the waves in LDS per document; capacities of 2^20 and more,
// whose room does not fit the packed key, take one wave over LDS-held fills
// with a maximum of the fill and then a minimum of the bin.
// qknr_bfd_emit_kernel: one workgroup per document and per bin filler writes
// its position ids and its cu_seqlens entry.
constexpr int kBfdMaxBins = 4096;
constexpr int kBfdThreads = 1024;
constexpr int kBfdLdsKeys = 2048;   // sorts of up to this many keys run in LDS

// Maximum / minimum over the 64 lanes, every lane gets it: the butterfly of
// group_sum<64> (quad xors and row mirrors by DPP, then the 16- and 32-lane
// halves swapped) with max / min in place of the sum.
template <bool MAX> __device__ inline uint32_t wave_extreme(uint32_t v)
{
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    v = op(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
    v = op(v, (uint32_t)__builtin_amdgcn_ds_bpermute((int)((threadIdx.x & 63) ^ 32) << 2, (int)v));
    return v;
}

// Minimum over the 64 lanes as a scalar: the butterfly of wave_extreme within
// each row of 16, then row broadcasts (lane 15 of rows 0 and 2 into rows 1 and
// 3; lane 31 into rows 2 and 3), which leave the minimum of the wave in lane 63.
__device__ inline uint32_t wave_min_scalar(uint32_t v)
{
    auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
    v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0xB1, 0xF, 0xF, false));
    v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x4E, 0xF, 0xF, false));
    v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x141, 0xF, 0xF, false));
    v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x140, 0xF, 0xF, false));
    v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false));
    v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

struct BfdWork {
    uint64_t *keys;     // [npow2]
    int32_t *rank;      // [n] placement order of each document within its bin
    int32_t *fill;      // [max_bins]
    int32_t *ndoc;      // [max_bins] documents per bin
    int32_t *first;     // [max_bins] index of the bin's first segment
};

// S: bins per lane held in registers while one wave places (64 S bins; the
// loop over them is straight-line code, which stops paying off beyond a few
// slots), 0 for bins in LDS.  BPT > 0: the whole workgroup places instead, BPT
// bins per thread (1024 BPT bins).  The launch picks S = 1 for up to 64 bins,
// else BPT = 1, 2 or 4.
template <int S, int BPT>
__global__ __launch_bounds__(kBfdThreads) void qknr_bfd_place_kernel(
    const int32_t *__restrict__ len, int n, int npow2, int cap, int max_bins, BfdWork w,
    int32_t *__restrict__ doc_start, int32_t *__restrict__ cu, int32_t *__restrict__ counts,
    int32_t *__restrict__ status)
{
    __shared__ int4 fill4[kBfdMaxBins / 4];  // bin fills, read four at a time
    __shared__ int32_t ndoc[kBfdMaxBins];
    __shared__ uint64_t lkeys[kBfdLdsKeys];  // the sort, when the keys fit
    __shared__ int32_t bad;
    int32_t *const fill = reinterpret_cast<int32_t *>(fill4);
    const int t = threadIdx.x;
    if (t == 0)
        bad = 0;
    __syncthreads();
    for (int i = t; i < n; i += kBfdThreads)
        if (len[i] < 1 || len[i] > cap)
            bad = 1;
    for (int i = t; i < npow2; i += kBfdThreads)
        w.keys[i] = i < n ? ((uint64_t)(uint32_t)(cap - len[i]) << 32) | (uint32_t)i : ~0ull;
    __syncthreads();
    if (bad) {
        if (t == 0) {
            status[0] = 2;
            counts[0] = counts[1] = 0;
        }
        return;
    }
    // bitonic sort, ascending, in LDS when the keys fit, else in the workspace
    uint64_t *const keys = npow2 <= kBfdLdsKeys ? lkeys : w.keys;
    if (keys == lkeys) {
        for (int i = t; i < npow2; i += kBfdThreads)
            lkeys[i] = w.keys[i];
        __syncthreads();
    }
    for (int k = 2; k <= npow2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = t; i < npow2; i += kBfdThreads) {
                const int l = i ^ j;
                if (l > i) {
                    const uint64_t a = keys[i], b = keys[l];
                    const bool up = (i & k) == 0;
                    if (up ? a > b : a < b) {
                        keys[i] = b;
                        keys[l] = a;
                    }
                }
            }
            __syncthreads();
        }
    }
    if constexpr (BPT > 0) {
        if (cap < (1 << 20)) {
            // Placement by the whole workgroup: thread t holds bins t + 1024 q
            // (fill and document count) in registers.  Each document is one
            // minimum of (room << 12 | bin) over the bins that fit: a DPP
            // minimum per wave, then the 16 waves' minima through LDS
            // (double-buffered, so one barrier per document); the least room,
            // lowest bin among equals, as in the single-wave loop.  The sorted
            // keys are staged 1024 at a time.
            constexpr int kW = kBfdThreads / 64;
            __shared__ uint32_t wmin[2][kW];
            __shared__ uint64_t kst[kBfdThreads];
            const int wave = t >> 6, lane = t & 63;
            int bf[BPT], bc[BPT];
#pragma unroll
            for (int q = 0; q < BPT; ++q)
                bf[q] = bc[q] = 0;
            int nb = 0, st = 0;
            for (int r = 0; r < n; ++r) {
                if ((r & (kBfdThreads - 1)) == 0) {
                    __syncthreads();  // the previous chunk's reads are done
                    kst[t] = r + t < n ? keys[r + t] : ~0ull;
                    __syncthreads();
                }
                const uint64_t key = kst[r & (kBfdThreads - 1)];
                const int i = (int)(uint32_t)key, L = cap - (int)(key >> 32);
                uint32_t cand = 0xffffffffu;
#pragma unroll
                for (int q = 0; q < BPT; ++q) {
                    const uint32_t bin = (uint32_t)(t + kBfdThreads * q);
                    const uint32_t room = (uint32_t)(cap - bf[q]);
                    const uint32_t k = (room << 12) | bin;
                    if (bin < (uint32_t)nb && room >= (uint32_t)L && k < cand)
                        cand = k;
                }
                const uint32_t m = wave_min_scalar(cand);
                if (lane == 0)
                    wmin[r & 1][wave] = m;
                __syncthreads();
                uint32_t g = 0xffffffffu;
#pragma unroll
                for (int v = 0; v < kW; ++v)
                    g = wmin[r & 1][v] < g ? wmin[r & 1][v] : g;
                int b, f0;
                if (g != 0xffffffffu) {
                    b = (int)(g & 0xfffu);
                    f0 = cap - (int)(g >> 12);
                } else {
                    if (nb == max_bins) {
                        st = 1;
                        break;
                    }
                    b = nb++;
                    f0 = 0;
                }
                if (t == (b & (kBfdThreads - 1))) {
                    const int qb = b / kBfdThreads;
#pragma unroll
                    for (int q = 0; q < BPT; ++q) {
                        if (q == qb) {
                            doc_start[i] = b * cap + f0;
                            w.rank[i] = bc[q];
                            bf[q] = f0 + L;
                            bc[q] += 1;
                        }
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < BPT; ++q) {
                const int bin = t + kBfdThreads * q;
                if (bin < nb) {
                    fill[bin] = bf[q];
                    ndoc[bin] = bc[q];
                }
            }
            __syncthreads();
            if (t == 0) {
                if (st) {
                    status[0] = 1;
                    counts[0] = counts[1] = 0;
                    return;
                }
                int seg = 0;
                for (int b = 0; b < nb; ++b) {
                    w.first[b] = seg;
                    w.fill[b] = fill[b];
                    w.ndoc[b] = ndoc[b];
                    seg += ndoc[b] + (fill[b] < cap ? 1 : 0);
                }
                cu[seg] = nb * cap;
                counts[0] = nb;
                counts[1] = seg;
                status[0] = 0;
            }
            return;
        }
    }
    if (t >= 64)
        return;  // placement: one wave
    const int lane = t;
    int nb = 0, st = 0;
    // (room << 12 | bin) orders by room, then bin, in 32 bits when room < 2^20
    const bool packed = cap < (1 << 20);
    // Documents are placed 64 at a time: the batch's sorted keys sit one per
    // lane, and lane j keeps document r0 + j's start and rank until the batch
    // is stored at once (a store per document would make every load of the
    // loop wait for it).
    uint64_t kbatch = 0;
    int my_doc = -1, my_start = 0, my_rank = 0;
    if (S > 0 && packed) {
        // The bins live in registers: bin 64 q + lane is slot q of lane `lane`
        // (fill and document count), so a placement reads no memory (64 S >=
        // max_bins).
        int32_t rf[S > 0 ? S : 1], rn[S > 0 ? S : 1];
#pragma unroll
        for (int q = 0; q < S; ++q)
            rf[q] = rn[q] = 0;
        for (int r = 0; r < n; ++r) {
            if ((r & 63) == 0) {
                if (my_doc >= 0) {
                    doc_start[my_doc] = my_start;
                    w.rank[my_doc] = my_rank;
                }
                my_doc = -1;
                kbatch = r + lane < n ? keys[r + lane] : ~0ull;
            }
            const int i = __builtin_amdgcn_readlane((int)(uint32_t)kbatch, r & 63);
            const int L = cap - __builtin_amdgcn_readlane((int)(uint32_t)(kbatch >> 32), r & 63);
            // the least room that fits (open bins hold at least one token),
            // lowest index among equals: one minimum of (room << 12 | bin)
            uint32_t best = 0xffffffffu;
            int bestn = 0;
#pragma unroll
            for (int q = 0; q < S; ++q) {
                const uint32_t bin = (uint32_t)(64 * q + lane);
                const uint32_t room = (uint32_t)(cap - rf[q]);
                const uint32_t key = (room << 12) | bin;
                const bool ok = bin < (uint32_t)nb && room >= (uint32_t)L && key < best;
                best = ok ? key : best;
                bestn = ok ? rn[q] : bestn;
            }
            const uint32_t m = wave_min_scalar(best);
            int b, f0, k0;
            if (m != 0xffffffffu) {
                b = (int)(m & 0xfffu);
                f0 = cap - (int)(m >> 12);
                k0 = __builtin_amdgcn_readlane(bestn, b & 63);  // the lane that holds bin b
            } else {
                if (nb == max_bins) {
                    st = 1;
                    break;
                }
                b = nb++;
                f0 = k0 = 0;
            }
            if (lane == (r & 63)) {
                my_doc = i;
                my_start = b * cap + f0;
                my_rank = k0;
            }
            const int qb = b >> 6;
            const bool mine = lane == (b & 63);
#pragma unroll
            for (int q = 0; q < S; ++q) {
                rf[q] = mine && q == qb ? f0 + L : rf[q];
                rn[q] = mine && q == qb ? k0 + 1 : rn[q];
            }
        }
        // the bins to LDS for the per-bin outputs
#pragma unroll
        for (int q = 0; q < S; ++q) {
            if (64 * q + lane < nb) {
                fill[64 * q + lane] = rf[q];
                ndoc[64 * q + lane] = rn[q];
            }
        }
        __builtin_amdgcn_wave_barrier();
    } else {
        for (int r = 0; r < n; ++r) {
            if ((r & 63) == 0) {
                if (my_doc >= 0) {
                    doc_start[my_doc] = my_start;
                    w.rank[my_doc] = my_rank;
                }
                my_doc = -1;
                kbatch = r + lane < n ? keys[r + lane] : ~0ull;
            }
            // the document's key as scalars, from the lane that holds it
            const int i = __builtin_amdgcn_readlane((int)(uint32_t)kbatch, r & 63);
            const int L = cap - __builtin_amdgcn_readlane((int)(uint32_t)(kbatch >> 32), r & 63);
            // this lane's bins lane, lane + 64, ...: the most filled that fits
            // (open bins hold at least one token, so 0 means none), lowest index
            // first; then the wave's most filled, and the lowest index holding it
            uint32_t wf, wb;
            if (packed) {
                // one minimum of (room << 12 | bin) over the bins that fit
                uint32_t best = 0xffffffffu;
                for (int q = lane; 4 * q < nb; q += 64) {
                    const int4 f4 = fill4[q];
                    const int fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t room = (uint32_t)(cap - fv[m]), b4 = (uint32_t)(4 * q + m);
                        const uint32_t key = (room << 12) | b4;
                        if (b4 < (uint32_t)nb && room >= (uint32_t)L && key < best)
                            best = key;
                    }
                }
                const uint32_t m = wave_min_scalar(best);
                wf = m == 0xffffffffu ? 0u : (uint32_t)cap - (m >> 12);
                wb = m & 0xfffu;
            } else {
                uint32_t bf = 0, bb = 0xffffffffu;
                for (int q = lane; 4 * q < nb; q += 64) {
                    const int4 f4 = fill4[q];   // bins 4q .. 4q + 3 (entries past nb are ignored)
                    const int fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int f = fv[m];
                        if (4 * q + m < nb && cap - f >= L && (uint32_t)f > bf) {
                            bf = (uint32_t)f;
                            bb = (uint32_t)(4 * q + m);
                        }
                    }
                }
                wf = wave_extreme<true>(bf);
                wb = wave_extreme<false>(bf == wf ? bb : 0xffffffffu);
            }
            int b, f0, k0;
            if (wf) {
                b = (int)wb;
                f0 = (int)wf;
                k0 = ndoc[b];
            } else {
                if (nb == max_bins) {
                    st = 1;
                    break;
                }
                b = nb++;
                f0 = k0 = 0;
            }
            if (lane == (r & 63)) {
                my_doc = i;
                my_start = b * cap + f0;
                my_rank = k0;
            }
            // lane 0 updates the bin; a wave's LDS accesses execute in order
            if (lane == 0) {
                fill[b] = f0 + L;
                ndoc[b] = k0 + 1;
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    if (!st && my_doc >= 0) {
        doc_start[my_doc] = my_start;
        w.rank[my_doc] = my_rank;
    }
    if (lane == 0) {
        if (st) {
            status[0] = 1;
            counts[0] = counts[1] = 0;
            return;
        }
        int seg = 0;
        for (int b = 0; b < nb; ++b) {
            w.first[b] = seg;
            w.fill[b] = fill[b];
            w.ndoc[b] = ndoc[b];
            seg += ndoc[b] + (fill[b] < cap ? 1 : 0);
        }
        cu[seg] = nb * cap;
        counts[0] = nb;
        counts[1] = seg;
        status[0] = 0;
    }
}

__global__ __launch_bounds__(256) void qknr_bfd_emit_kernel(
    const int32_t *__restrict__ len, int n, int cap, BfdWork w,
    const int32_t *__restrict__ doc_start, int32_t *__restrict__ pos, int32_t *__restrict__ cu,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ status)
{
    if (status[0] != 0)
        return;
    const int x = blockIdx.x, t = threadIdx.x;
    int start, count, seg;
    if (x < n) {
        start = doc_start[x];
        count = len[x];
        seg = w.first[start / cap] + w.rank[x];
    } else {
        const int b = x - n;
        if (b >= counts[0])
            return;
        const int f = w.fill[b];
        if (f >= cap)
            return;
        start = b * cap + f;
        count = cap - f;
        seg = w.first[b] + w.ndoc[b];
    }
    if (t == 0)
        cu[seg] = start;
    for (int i = t; i < count; i += 256)
        pos[start + i] = i;
}

// dst = a ^ b: two read streams and one write stream, the backward's shape
// ---- host side ---------------------------------------------------------------

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Rows per group for a dtype and head_dim: 64 lanes / (head_dim / E lanes per row).
inline int rows_per_group(qknr_dtype dt, int head_dim)
{
    const int E = dt == QKNR_BF16 ? 8 : 4;
    return 64 / (head_dim / E);
}

struct Plan {
    int tb_tokens;
    int groups;
    int64_t token_blocks;
};

Plan make_plan(int64_t tokens, int hq, int hkv, int head_dim, int rotary_dim, qknr_dtype dt)
{
    Plan pl;
    const int rw = rows_per_group(dt, head_dim);
    const int rpt = hq + hkv;
    const int h = rotary_dim / 2;
    const int cap = 256;  // cos/sin table entries per wave: tokens * head_dim / 2 <= cap
    pl.tb_tokens = rpt >= rw ? 1 : rw / rpt;
    // Take more tokens per block while their cos/sin evaluations leave lanes of
    // the wave idle and the table has room.
    while (h > 0 && pl.tb_tokens * h < QKNR_MIN_COS_SIN_PER_BLOCK &&
           2 * pl.tb_tokens * (head_dim / 2) <= cap)
        pl.tb_tokens *= 2;
    pl.groups = (pl.tb_tokens * rpt + rw - 1) / rw;
    pl.token_blocks = (tokens + pl.tb_tokens - 1) / pl.tb_tokens;
    return pl;
}

// Workgroups of a persistent launch: one per 4 token blocks, at most what the
// device keeps resident at once (CUs x resident workgroups per CU for this
// kernel, queried once per device and kernel), and at most `cap`.
constexpr int kMaxDevices = 64;

struct ResidentCache {
    std::atomic<int> v[kMaxDevices];
};

// Resident workgroups of a kernel with dynamic LDS, per device and LDS size:
// a few sizes per process, kept in a small table (computed uncached once it
// is full).
struct ResidentCacheLds {
    struct Entry {
        int dev;
        size_t lds;
        int v;
    };
    std::mutex m;
    Entry e[16];
    int n = 0;
};

template <typename Kernel>
hipError_t resident_workgroups_lds(Kernel kernel, ResidentCacheLds &cache, size_t lds, int *out,
                                   int threads)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    {
        std::lock_guard<std::mutex> g(cache.m);
        for (int i = 0; i < cache.n; ++i)
            if (cache.e[i].dev == dev && cache.e[i].lds == lds) {
                *out = cache.e[i].v;
                return hipSuccess;
            }
    }
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
    if (e != hipSuccess)
        return e;
    const int v = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    {
        std::lock_guard<std::mutex> g(cache.m);
        if (cache.n < 16)
            cache.e[cache.n++] = {dev, lds, v};
    }
    *out = v;
    return hipSuccess;
}

template <typename Kernel>
hipError_t resident_workgroups(Kernel kernel, ResidentCache &cache, int *out,
                               int threads = kThreads)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cache.v[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return hipSuccess;
        }
    }
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    if (e != hipSuccess)
        return e;
    const int v = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    if (dev >= 0 && dev < kMaxDevices)
        cache.v[dev].store(v, std::memory_order_relaxed);
    *out = v;
    return hipSuccess;
}

// Waves take token blocks round-robin, so the launch lasts as long as the
// busiest wave.  Use the fewest waves that still give every wave the same
// number of blocks as the widest resident launch would (at most one fewer).
int64_t grid_size(const Plan &pl, int resident, int64_t cap)
{
    int64_t max_wg = resident < cap ? resident : cap;
    if (max_wg < 1)
        max_wg = 1;
    const int64_t per_wave = (pl.token_blocks + max_wg * kWaves - 1) / (max_wg * kWaves);
    const int64_t waves = (pl.token_blocks + per_wave - 1) / per_wave;
    const int64_t wg = (waves + kWaves - 1) / kWaves;
    return wg < 1 ? 1 : wg;
}

// The forward's grid.  A persistent grid (grid_size) gives every wave the same
// share of token blocks, but waves stream at different rates (per-wave exit
// times spread over ~20% of a launch), so the launch lasts as long as its
// slowest wave.  When a wave's share is long (at least kOversubStages stages),
// short shares of at least kOversubMinStages stages (whole token blocks) in
// many rounds of workgroups let the dispatcher fill the CUs that finish
// first; short persistent shares stay as they are, where more rounds would
// cost more set-up than they balance.
constexpr int kOversubStages = 16;
constexpr int kOversubMinStages = 4;
constexpr int64_t kMaxOversubBlocks = 1 << 20;

int64_t grid_size_fwd(const Plan &pl, int resident, int64_t cap)
{
    const int64_t wg = grid_size(pl, resident, cap);
    const int64_t per_wave = (pl.token_blocks + wg * kWaves - 1) / (wg * kWaves);
    const int64_t nbatch = (pl.groups + kFwdUnroll - 1) / kFwdUnroll;
    if (per_wave * nbatch < kOversubStages)
        return wg;
    const int64_t bpw = (kOversubMinStages + nbatch - 1) / nbatch;  // blocks per wave
    const int64_t waves = (pl.token_blocks + bpw - 1) / bpw;
    const int64_t n = (waves + kWaves - 1) / kWaves;
    return n < kMaxOversubBlocks ? n : kMaxOversubBlocks;
}

int64_t max_bwd_blocks(const Plan &pl)
{
    const int64_t b = (pl.token_blocks + kWaves - 1) / kWaves;
    return b < kMaxBwdBlocks ? b : kMaxBwdBlocks;
}

constexpr uint32_t kKnownFlags = QKNR_FLAG_INTERLEAVED | QKNR_FLAG_FREQ_HEAD_DIM |
                                  QKNR_FLAG_NO_WEIGHT | QKNR_FLAG_LAYERNORM |
                                  QKNR_FLAG_HEAD_WEIGHTS;

qknr_status check_common(const void *q, const void *k, const void *wq, const void *wk,
                         const int32_t *pos, int64_t tokens, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                         qknr_dtype dtype, uint32_t flags)
{
    if (tokens < 0 || hq < 1 || hkv < 1 || hq > kMaxHeads || hkv > kMaxHeads)
        return QKNR_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps) || !(theta > 0.0) || !isfinite(theta))
        return QKNR_ERR_INVALID_ARG;
    if ((flags & ~kKnownFlags) != 0)
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
    const bool has_w = (flags & QKNR_FLAG_NO_WEIGHT) == 0;
    if (!q || !k || !pos || (has_w && (!wq || !wk)))
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(pos, 4))
        return QKNR_ERR_MISALIGNED;
    if (has_w && (!aligned(wq, 16) || !aligned(wk, 16)))
        return QKNR_ERR_MISALIGNED;
    return QKNR_OK;
}

// A token stride: at least the token's rows, at most 2^40 elements, and whole
// 16-byte chunks so every lane's chunk stays aligned.
qknr_status check_stride(int64_t stride, int32_t heads, int32_t head_dim, qknr_dtype dtype)
{
    const int64_t chunk = dtype == QKNR_BF16 ? 8 : 4;
    if (stride < (int64_t)heads * head_dim || stride > ((int64_t)1 << 40))
        return QKNR_ERR_INVALID_ARG;
    if (stride % chunk != 0)
        return QKNR_ERR_MISALIGNED;
    return QKNR_OK;
}

qknr_layout dense_layout(int32_t hq, int32_t hkv, int32_t head_dim)
{
    qknr_layout l;
    l.q_stride = l.q_out_stride = l.dq_out_stride = (int64_t)hq * head_dim;
    l.k_stride = l.k_out_stride = l.dk_out_stride = (int64_t)hkv * head_dim;
    l.k_out_slots = nullptr;
    l.k_out_rows = 0;
    return l;
}

// Everything an entry point passes beyond the plain arguments.  The plain and
// _ex entry points fill it with defaults (no biases, the theta formula, no
// attention factor).
struct Options {
    uint32_t flags;
    qknr_layout layout;
    const void *bq, *bk;      // forward biases, or null
    const double *inv_freq;   // host table of rotary_dim / 2 frequencies, or null
    double attn;              // factor on cos and sin
    int32_t gq, gk;           // heads per norm group
    bool grouped() const { return gq > 1 || gk > 1 || (flags & QKNR_FLAG_HEAD_WEIGHTS) != 0; }
};

Options make_options(uint32_t flags, const qknr_layout *layout, int32_t hq, int32_t hkv,
                     int32_t head_dim)
{
    Options o;
    o.flags = flags;
    o.layout = layout ? *layout : dense_layout(hq, hkv, head_dim);
    o.bq = o.bk = nullptr;
    o.inv_freq = nullptr;
    o.attn = 1.0;
    o.gq = o.gk = 1;
    return o;
}

// The shape arguments that bound what options_from reads from the caller's
// frequency table (rotary_dim / 2 entries), checked before it reads them.
qknr_status check_shape(int32_t head_dim, int32_t rotary_dim, qknr_dtype dtype)
{
    if (dtype != QKNR_F32 && dtype != QKNR_BF16)
        return QKNR_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return QKNR_ERR_UNSUPPORTED;
    if (rotary_dim < 0 || rotary_dim > head_dim || rotary_dim % 16 != 0)
        return QKNR_ERR_UNSUPPORTED;
    return QKNR_OK;
}

// Checks the options shared by the forward and the backward; converts the
// public struct (a null pointer means all defaults).  The caller has checked
// the shape (check_shape), which bounds the table read here.
qknr_status options_from(const qknr_options *opt, int32_t hq, int32_t hkv, int32_t head_dim,
                         int32_t rotary_dim, Options *o)
{
    *o = make_options(opt ? opt->flags : 0u, opt ? opt->layout : nullptr, hq, hkv, head_dim);
    if (!opt)
        return QKNR_OK;
    if ((opt->bq == nullptr) != (opt->bk == nullptr))
        return QKNR_ERR_INVALID_ARG;
    if (opt->bq && (!aligned(opt->bq, 16) || !aligned(opt->bk, 16)))
        return QKNR_ERR_MISALIGNED;
    o->bq = opt->bq;
    o->bk = opt->bk;
    const double a = opt->attention_factor;
    if (!isfinite(a))
        return QKNR_ERR_INVALID_ARG;
    o->attn = a == 0.0 ? 1.0 : a;
    if (opt->inv_freq) {
        for (int i = 0; i < rotary_dim / 2; ++i)
            if (!isfinite(opt->inv_freq[i]))
                return QKNR_ERR_INVALID_ARG;
        o->inv_freq = opt->inv_freq;
    }
    o->gq = opt->norm_group_q == 0 ? 1 : opt->norm_group_q;
    o->gk = opt->norm_group_k == 0 ? 1 : opt->norm_group_k;
    if (o->gq < 1 || o->gk < 1 || (hq > 0 && hq % o->gq != 0) || (hkv > 0 && hkv % o->gk != 0))
        return QKNR_ERR_INVALID_ARG;
    return QKNR_OK;
}

void fill_params(Params &p, const Plan &pl, const void *q, const void *k, const void *wq,
                 const void *wk, const int32_t *pos, int64_t tokens, int32_t hq, int32_t hkv,
                 int32_t head_dim, int32_t rotary_dim, float eps, double theta, const Options &o)
{
    const qknr_layout &l = o.layout;
    memset(&p, 0, sizeof p);
    p.x[0] = q;
    p.x[1] = k;
    p.has_w = (o.flags & QKNR_FLAG_NO_WEIGHT) ? 0 : 1;
    p.w[0] = p.has_w ? wq : nullptr;
    p.w[1] = p.has_w ? wk : nullptr;
    p.b[0] = o.bq;
    p.b[1] = o.bk;
    p.has_b = o.bq ? 1 : 0;
    p.layernorm = (o.flags & QKNR_FLAG_LAYERNORM) ? 1 : 0;
    p.group[0] = o.gq;
    p.group[1] = o.gk;
    p.head_w = (o.flags & QKNR_FLAG_HEAD_WEIGHTS) ? 1 : 0;
    p.stages = 1;
    p.attn = o.attn;
    p.pos = pos;
    p.slots = l.k_out_slots;
    p.k_out_rows = l.k_out_slots ? l.k_out_rows : 0;
    p.xs[0] = l.q_stride;
    p.xs[1] = l.k_stride;
    p.os[0] = l.q_out_stride;
    p.os[1] = l.k_out_stride;
    p.ds[0] = l.dq_out_stride;
    p.ds[1] = l.dk_out_stride;
    p.tokens = tokens;
    p.token_blocks = pl.token_blocks;
    p.heads[0] = hq;
    p.heads[1] = hkv;
    p.rows_per_token = hq + hkv;
    p.inv_rows_per_token = 1.0f / (float)(hq + hkv);
    p.tb_tokens = pl.tb_tokens;
    p.groups = pl.groups;
    p.rotary_dim = rotary_dim;
    p.eps = eps;
    // RoPE frequencies theta^(-2i/d) in fp64 (Rope to Nope and Back Again,
    // abstract: RoPE), d the rotated width R (Partial RoPE abstract) or, on
    // request, the head width; or the caller's table (the same abstract's
    // "extensions" of RoPE change these frequencies).
    const double denom = (o.flags & QKNR_FLAG_FREQ_HEAD_DIM) ? head_dim : rotary_dim;
    for (int i = 0; i < rotary_dim / 2; ++i)
        p.inv_freq[i] = o.inv_freq ? o.inv_freq[i] : pow(theta, -2.0 * (double)i / denom);
}

template <typename IO, int D, bool IL, bool SLOT, bool EXT>
hipError_t launch_fwd(const Params &p, const Plan &pl, hipStream_t s)
{
    static ResidentCache cache;
    auto kernel = qknr_kernel<IO, D, kFwdUnroll, false, IL, SLOT, EXT>;
    int resident = 0;
    hipError_t e = resident_workgroups(kernel, cache, &resident);
    if (e != hipSuccess)
        return e;
    const int64_t blocks = grid_size_fwd(pl, resident, kMaxFwdBlocks);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// The gradients the backward writes after its main kernel.
struct Grads {
    void *dwq, *dwk, *dbq, *dbk;
};

template <typename IO, int D, bool IL, bool EXT>
hipError_t launch_bwd(const Params &p, const Plan &pl, const Grads &gr, hipStream_t s)
{
    static ResidentCache cache;
    auto kernel = qknr_kernel<IO, D, kBwdUnroll, true, IL, false, EXT>;
    int resident = 0;
    hipError_t e = resident_workgroups(kernel, cache, &resident);
    if (e != hipSuccess)
        return e;
    const int64_t blocks = grid_size(pl, resident, kMaxBwdBlocks);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    void *dwq = p.has_w ? gr.dwq : nullptr, *dwk = p.has_w ? gr.dwk : nullptr;
    void *dbq = p.has_b ? gr.dbq : nullptr, *dbk = p.has_b ? gr.dbk : nullptr;
    if (e != hipSuccess || (!dwq && !dbq))
        return e;
    constexpr int kColsPerBlock = kFinalizeThreads / 64;
    const int cols = (p.has_b ? 4 : 2) * D;
    const GradCols gc = {{dwq, dwk, dbq, dbk}, {D, D}};
    hipLaunchKernelGGL((qknr_dw_finalize_kernel<IO>), dim3((cols + kColsPerBlock - 1) / kColsPerBlock),
                       dim3(kFinalizeThreads), 0, s, (const float *)p.partials, (int)blocks, cols, gc);
    return hipGetLastError();
}

template <typename IO, int D, bool EXT>
hipError_t fwd_variant(const Params &p, const Plan &pl, bool il, bool slot, hipStream_t s)
{
    if (il)
        return slot ? launch_fwd<IO, D, true, true, EXT>(p, pl, s)
                    : launch_fwd<IO, D, true, false, EXT>(p, pl, s);
    return slot ? launch_fwd<IO, D, false, true, EXT>(p, pl, s)
                : launch_fwd<IO, D, false, false, EXT>(p, pl, s);
}

template <typename IO, bool EXT>
hipError_t fwd_dispatch(const Params &p, const Plan &pl, int head_dim, bool il, bool slot,
                        hipStream_t s)
{
    return head_dim == 64 ? fwd_variant<IO, 64, EXT>(p, pl, il, slot, s)
         : head_dim == 128 ? fwd_variant<IO, 128, EXT>(p, pl, il, slot, s)
                           : fwd_variant<IO, 256, EXT>(p, pl, il, slot, s);
}

template <typename IO, int D, bool EXT>
hipError_t bwd_variant(const Params &p, const Plan &pl, bool il, const Grads &gr, hipStream_t s)
{
    return il ? launch_bwd<IO, D, true, EXT>(p, pl, gr, s)
              : launch_bwd<IO, D, false, EXT>(p, pl, gr, s);
}

template <typename IO, bool EXT>
hipError_t bwd_dispatch(const Params &p, const Plan &pl, int head_dim, bool il, const Grads &gr,
                        hipStream_t s)
{
    return head_dim == 64 ? bwd_variant<IO, 64, EXT>(p, pl, il, gr, s)
         : head_dim == 128 ? bwd_variant<IO, 128, EXT>(p, pl, il, gr, s)
                           : bwd_variant<IO, 256, EXT>(p, pl, il, gr, s);
}

// ---- launches of the norm-group kernel ----

// Tokens per iteration of qknr_group_kernel: as many whole tokens as fit in
// the workgroup's chunk slots and the cos/sin table; 0 when a token does not
// fit.
int group_tpi(int32_t hq, int32_t hkv, int32_t head_dim, int32_t rotary_dim, qknr_dtype dt,
              bool bwd, bool head_w)
{
    const int E = dt == QKNR_BF16 ? 8 : 4;
    const int64_t n = (int64_t)(hq + hkv) * (head_dim / E);
    const int64_t cap = (int64_t)group_threads(bwd) * group_slots(bwd, E);
    if (n > cap)
        return 0;
    (void)head_w;
    int64_t tpi = cap / n;
    const int h = rotary_dim / 2;
    if (h > 0 && tpi * h > kGroupMaxCosSin)
        tpi = kGroupMaxCosSin / h;
    return (int)(tpi < 1 ? 1 : tpi);
}

// Dynamic LDS of qknr_group_kernel: the weight chunks and, in the forward,
// the bias chunks, 16 bytes each, for every head ([H, D]) or per tensor ([D]).
size_t group_lds_bytes(const Params &p, int chunks_per_row, bool bwd)
{
    const int wrows = p.head_w ? p.heads[0] + p.heads[1] : 2;
    const int sets = (p.has_w ? 1 : 0) + (!bwd && p.has_b ? 1 : 0);
    return (size_t)sets * (size_t)wrows * (size_t)chunks_per_row * 16u;
}

// Shape of qknr_gwave_kernel for these sizes: tokens per block and stages
// per token ({0, 0}: it does not apply).  A stage is two wave instructions of
// rows.  Either a block of whole tokens fits one stage (and its cos/sin the
// wave's table), or a token spans up to kGwMaxStages stages and every norm
// group of q (gq heads) and of k (gk heads) lies within one of them.
struct GwaveShape {
    int tb, stages;
};

GwaveShape gwave_shape(int32_t hq, int32_t hkv, int32_t head_dim, qknr_dtype dt, int32_t gq,
                       int32_t gk)
{
    const int rpt = hq + hkv, sr = 2 * rows_per_group(dt, head_dim);
    if (rpt <= sr) {
        int tb = sr / rpt;
        while (tb > 1 && tb * (head_dim / 2) > 256)
            --tb;
        return {tb, 1};
    }
    const int st = (rpt + sr - 1) / sr;
    if (st > kGwMaxStages)
        return {0, 0};
    for (int g = 0; g < hq; g += gq)
        if (g / sr != (g + gq - 1) / sr)
            return {0, 0};
    for (int g = hq; g < rpt; g += gk)
        if (g / sr != (g + gk - 1) / sr)
            return {0, 0};
    return {1, st};
}

Plan gwave_plan(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim, qknr_dtype dt,
                GwaveShape sh)
{
    Plan pl;
    const int rw = rows_per_group(dt, head_dim);
    pl.tb_tokens = sh.tb;
    pl.groups = (sh.tb * (hq + hkv) + rw - 1) / rw;
    pl.token_blocks = (tokens + sh.tb - 1) / sh.tb;
    return pl;
}

// Workgroups of a qknr_gwave_kernel launch: as qknr_kernel's for the (token
// block, stage) pairs, then a multiple of the waves per stage set (m
// workgroups hold a whole number of stage sets); at most gwave_max_blocks.
int64_t gwave_round(int64_t blocks, int stages)
{
    int g = stages, b = kWaves;
    while (b) {
        const int t = g % b;
        g = b;
        b = t;
    }
    const int64_t m = stages / g;
    return blocks >= m ? blocks / m * m : m;
}

int64_t gwave_max_blocks(const Plan &pl, int stages)
{
    Plan pw = pl;
    pw.token_blocks = pl.token_blocks * stages;
    const int64_t b = max_bwd_blocks(pw), r = gwave_round(b, stages);
    return r > b ? r : b;
}

// Backward workgroups of the norm-group kernel (= partial rows).
int64_t group_blocks(int64_t tokens, int tpi)
{
    const int64_t iters = (tokens + tpi - 1) / tpi;
    return iters < kMaxBwdBlocks ? iters : kMaxBwdBlocks;
}

// Gradient columns of one partial row: dwq, dwk, dbq, dbk.
int64_t group_cols(int32_t hq, int32_t hkv, int32_t head_dim, bool head_w)
{
    return 2 * (head_w ? (int64_t)(hq + hkv) * head_dim : 2 * (int64_t)head_dim);
}

template <typename IO, int D, bool BWD, bool IL, bool SLOT>
hipError_t launch_group(const Params &p, int64_t max_blocks, const GradCols &gc, hipStream_t s)
{
    static ResidentCacheLds cache;
    auto kernel = qknr_group_kernel<IO, D, BWD, IL, SLOT>;
    const size_t lds = group_lds_bytes(p, D / Io<IO>::E, BWD);
    int resident = 0;
    hipError_t e = resident_workgroups_lds(kernel, cache, lds, &resident, group_threads(BWD));
    if (e != hipSuccess)
        return e;
    const int64_t iters = (p.tokens + p.tb_tokens - 1) / p.tb_tokens;
    int64_t blocks = iters < resident ? iters : resident;
    if (blocks > max_blocks)
        blocks = max_blocks;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(group_threads(BWD)), lds, s, p);
    e = hipGetLastError();
    if (!BWD || e != hipSuccess || (!gc.out[0] && !gc.out[2]))
        return e;
    const int cols = 2 * (gc.n[0] + gc.n[1]);
    hipLaunchKernelGGL((qknr_group_finalize_kernel<IO>),
                       dim3((cols + kGroupFinalizeCols - 1) / kGroupFinalizeCols),
                       dim3(kGroupFinalizeThreads), 0, s, (const float *)p.partials, (int)blocks,
                       cols, gc);
    return hipGetLastError();
}

template <typename IO, int D, bool BWD, bool IL, bool SLOT>
hipError_t launch_gwave(const Params &p, const Plan &pl, const GradCols &gc, hipStream_t s)
{
    static ResidentCache cache;
    auto kernel = qknr_gwave_kernel<IO, D, BWD, IL, SLOT>;
    int resident = 0;
    hipError_t e = resident_workgroups(kernel, cache, &resident);
    if (e != hipSuccess)
        return e;
    Plan pw = pl;
    pw.token_blocks = pl.token_blocks * p.stages;  // (token block, stage) pairs
    const int64_t blocks =
        gwave_round(grid_size(pw, resident, BWD ? kMaxBwdBlocks : kMaxFwdBlocks), p.stages);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (!BWD || e != hipSuccess || (!gc.out[0] && !gc.out[2]))
        return e;
    const int cols = 2 * (gc.n[0] + gc.n[1]);
    hipLaunchKernelGGL((qknr_group_finalize_kernel<IO>),
                       dim3((cols + kGroupFinalizeCols - 1) / kGroupFinalizeCols),
                       dim3(kGroupFinalizeThreads), 0, s, (const float *)p.partials, (int)blocks,
                       cols, gc);
    return hipGetLastError();
}

template <typename IO, bool BWD>
hipError_t gwave_dispatch(const Params &p, const Plan &pl, int head_dim, bool il,
                          const GradCols &gc, hipStream_t s)
{
    if constexpr (!BWD) {
        if (p.slots) {
            if (il)
                return head_dim == 64 ? launch_gwave<IO, 64, false, true, true>(p, pl, gc, s)
                     : head_dim == 128 ? launch_gwave<IO, 128, false, true, true>(p, pl, gc, s)
                                       : launch_gwave<IO, 256, false, true, true>(p, pl, gc, s);
            return head_dim == 64 ? launch_gwave<IO, 64, false, false, true>(p, pl, gc, s)
                 : head_dim == 128 ? launch_gwave<IO, 128, false, false, true>(p, pl, gc, s)
                                   : launch_gwave<IO, 256, false, false, true>(p, pl, gc, s);
        }
    }
    if (il)
        return head_dim == 64 ? launch_gwave<IO, 64, BWD, true, false>(p, pl, gc, s)
             : head_dim == 128 ? launch_gwave<IO, 128, BWD, true, false>(p, pl, gc, s)
                               : launch_gwave<IO, 256, BWD, true, false>(p, pl, gc, s);
    return head_dim == 64 ? launch_gwave<IO, 64, BWD, false, false>(p, pl, gc, s)
         : head_dim == 128 ? launch_gwave<IO, 128, BWD, false, false>(p, pl, gc, s)
                           : launch_gwave<IO, 256, BWD, false, false>(p, pl, gc, s);
}

template <typename IO, bool BWD>
hipError_t group_dispatch(const Params &p, int head_dim, bool il, int64_t max_blocks,
                          const GradCols &gc, hipStream_t s)
{
    if constexpr (!BWD) {
        if (p.slots) {
            if (il)
                return head_dim == 64 ? launch_group<IO, 64, false, true, true>(p, max_blocks, gc, s)
                     : head_dim == 128 ? launch_group<IO, 128, false, true, true>(p, max_blocks, gc, s)
                                       : launch_group<IO, 256, false, true, true>(p, max_blocks, gc, s);
            return head_dim == 64 ? launch_group<IO, 64, false, false, true>(p, max_blocks, gc, s)
                 : head_dim == 128 ? launch_group<IO, 128, false, false, true>(p, max_blocks, gc, s)
                                   : launch_group<IO, 256, false, false, true>(p, max_blocks, gc, s);
        }
    }
    if (il)
        return head_dim == 64 ? launch_group<IO, 64, BWD, true, false>(p, max_blocks, gc, s)
             : head_dim == 128 ? launch_group<IO, 128, BWD, true, false>(p, max_blocks, gc, s)
                               : launch_group<IO, 256, BWD, true, false>(p, max_blocks, gc, s);
    return head_dim == 64 ? launch_group<IO, 64, BWD, false, false>(p, max_blocks, gc, s)
         : head_dim == 128 ? launch_group<IO, 128, BWD, false, false>(p, max_blocks, gc, s)
                           : launch_group<IO, 256, BWD, false, false>(p, max_blocks, gc, s);
}

qknr_status run_fwd(const void *q, const void *k, const void *wq, const void *wk,
                    const int32_t *pos, int64_t tokens, int32_t hq, int32_t hkv,
                    int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                    qknr_dtype dtype, const Options &o, void *q_out, void *k_out, void *stream)
{
    qknr_status st = check_common(q, k, wq, wk, pos, tokens, hq, hkv, head_dim, rotary_dim, eps,
                                  theta, dtype, o.flags);
    if (st != QKNR_OK || tokens == 0)
        return st;
    if (!q_out || !k_out)
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(q_out, 16) || !aligned(k_out, 16))
        return QKNR_ERR_MISALIGNED;
    const qknr_layout &l = o.layout;
    const int64_t st4[4] = {l.q_stride, l.k_stride, l.q_out_stride, l.k_out_stride};
    const int32_t hd4[4] = {hq, hkv, hq, hkv};
    for (int i = 0; i < 4; ++i)
        if ((st = check_stride(st4[i], hd4[i], head_dim, dtype)) != QKNR_OK)
            return st;
    if (l.k_out_slots && !aligned(l.k_out_slots, 8))
        return QKNR_ERR_MISALIGNED;
    if (l.k_out_slots && l.k_out_rows < 1)
        return QKNR_ERR_INVALID_ARG;
    const Plan pl = make_plan(tokens, hq, hkv, head_dim, rotary_dim, dtype);
    Params p;
    fill_params(p, pl, q, k, wq, wk, pos, tokens, hq, hkv, head_dim, rotary_dim, eps, theta, o);
    p.out[0] = q_out;
    p.out[1] = k_out;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool il = (o.flags & QKNR_FLAG_INTERLEAVED) != 0;
    const bool slot = l.k_out_slots != nullptr;
    if (o.grouped()) {
        const GradCols none = {{nullptr, nullptr, nullptr, nullptr}, {0, 0}};
        // norm groups / [H, D] weights: whole groups in a wave's stage, else
        // whole tokens per workgroup (whose limits bound both)
        const int tpi = group_tpi(hq, hkv, head_dim, rotary_dim, dtype, false, p.head_w != 0);
        if (tpi == 0)
            return QKNR_ERR_UNSUPPORTED;
        const GwaveShape sh = gwave_shape(hq, hkv, head_dim, dtype, o.gq, o.gk);
        if (sh.tb > 0) {
            const Plan gp = gwave_plan(tokens, hq, hkv, head_dim, dtype, sh);
            p.tb_tokens = gp.tb_tokens;
            p.groups = gp.groups;
            p.token_blocks = gp.token_blocks;
            p.stages = sh.stages;
            const hipError_t e = dtype == QKNR_BF16
                                     ? gwave_dispatch<Bf16, false>(p, gp, head_dim, il, none, s)
                                     : gwave_dispatch<float, false>(p, gp, head_dim, il, none, s);
            return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
        }
        p.tb_tokens = tpi;
        const hipError_t e = dtype == QKNR_BF16
                                 ? group_dispatch<Bf16, false>(p, head_dim, il, kMaxFwdBlocks, none, s)
                                 : group_dispatch<float, false>(p, head_dim, il, kMaxFwdBlocks, none, s);
        return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
    }
    // A few tokens whose rows span several wave stages (decode steps of wide
    // heads): the dense kernel walks each token's stages in one wave, one
    // after the other; the wave kernel with per-head norm groups (the same
    // arithmetic, bit for bit: a group of one row adds its own sum to +0 and
    // scales it by the exact 1 / D) gives each stage of a token its own wave.
    if (tokens <= kSplitTokens) {
        const GwaveShape sh = gwave_shape(hq, hkv, head_dim, dtype, 1, 1);
        if (sh.tb > 0 && sh.stages > 1) {
            const GradCols none = {{nullptr, nullptr, nullptr, nullptr}, {0, 0}};
            const Plan gp = gwave_plan(tokens, hq, hkv, head_dim, dtype, sh);
            p.tb_tokens = gp.tb_tokens;
            p.groups = gp.groups;
            p.token_blocks = gp.token_blocks;
            p.stages = sh.stages;
            const hipError_t e = dtype == QKNR_BF16
                                     ? gwave_dispatch<Bf16, false>(p, gp, head_dim, il, none, s)
                                     : gwave_dispatch<float, false>(p, gp, head_dim, il, none, s);
            return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
        }
    }
    const bool ext = p.layernorm || p.has_b;
    hipError_t e;
    if (dtype == QKNR_BF16)
        e = ext ? fwd_dispatch<Bf16, true>(p, pl, head_dim, il, slot, s)
                : fwd_dispatch<Bf16, false>(p, pl, head_dim, il, slot, s);
    else
        e = ext ? fwd_dispatch<float, true>(p, pl, head_dim, il, slot, s)
                : fwd_dispatch<float, false>(p, pl, head_dim, il, slot, s);
    return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

size_t bwd_workspace_bytes(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                           qknr_dtype dtype)
{
    if (tokens <= 0 || hq < 1 || hkv < 1 || (head_dim != 64 && head_dim != 128 && head_dim != 256) ||
        (dtype != QKNR_F32 && dtype != QKNR_BF16))
        return 0;
    // rotary_dim 0 gives the fewest tokens per block, hence the most workgroups:
    // an upper bound for every rotary_dim.  Four [D] columns sets per
    // workgroup: dwq, dwk and, with bias gradients, dbq, dbk.
    return (size_t)max_bwd_blocks(make_plan(tokens, hq, hkv, head_dim, 0, dtype)) * 4 *
           (size_t)head_dim * sizeof(float);
}

// Workspace of a backward with these options: the plain kernel's, or the
// norm-group kernel's partial rows.
size_t bwd_workspace_bytes_opt(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                               int32_t rotary_dim, qknr_dtype dtype, const Options &o)
{
    const size_t plain = bwd_workspace_bytes(tokens, hq, hkv, head_dim, dtype);
    if (!o.grouped() || plain == 0)
        return plain;
    const bool head_w = (o.flags & QKNR_FLAG_HEAD_WEIGHTS) != 0;
    const size_t cols = (size_t)group_cols(hq, hkv, head_dim, head_w);
    const int tpi = group_tpi(hq, hkv, head_dim, rotary_dim, dtype, true, head_w);
    if (tpi == 0)
        return 0;
    const GwaveShape sh = gwave_shape(hq, hkv, head_dim, dtype, o.gq, o.gk);
    if (sh.tb > 0)
        return (size_t)gwave_max_blocks(gwave_plan(tokens, hq, hkv, head_dim, dtype, sh),
                                        sh.stages) *
               cols * sizeof(float);
    return (size_t)group_blocks(tokens, tpi) * cols * sizeof(float);
}

qknr_status run_bwd(const void *q, const void *k, const void *wq, const void *wk,
                    const int32_t *pos, int64_t tokens, int32_t hq, int32_t hkv,
                    int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                    qknr_dtype dtype, const Options &o, const void *dq_out, const void *dk_out,
                    void *dq, void *dk, const Grads &gr, void *workspace, size_t workspace_bytes,
                    void *stream)
{
    qknr_status st = check_common(q, k, wq, wk, pos, tokens, hq, hkv, head_dim, rotary_dim, eps,
                                  theta, dtype, o.flags);
    if (st != QKNR_OK || tokens == 0)
        return st;
    const bool has_w = (o.flags & QKNR_FLAG_NO_WEIGHT) == 0;
    if (!dq_out || !dk_out || !dq || !dk || (has_w && (!gr.dwq || !gr.dwk)))
        return QKNR_ERR_INVALID_ARG;
    if ((gr.dbq == nullptr) != (gr.dbk == nullptr))
        return QKNR_ERR_INVALID_ARG;
    if (!aligned(dq_out, 16) || !aligned(dk_out, 16) || !aligned(dq, 16) || !aligned(dk, 16))
        return QKNR_ERR_MISALIGNED;
    if (has_w && (!aligned(gr.dwq, 16) || !aligned(gr.dwk, 16)))
        return QKNR_ERR_MISALIGNED;
    if (gr.dbq && (!aligned(gr.dbq, 16) || !aligned(gr.dbk, 16)))
        return QKNR_ERR_MISALIGNED;
    const qknr_layout &l = o.layout;
    if (l.k_out_slots)
        return QKNR_ERR_INVALID_ARG;
    const int64_t st6[6] = {l.q_stride,      l.k_stride,      l.q_out_stride,
                            l.k_out_stride,  l.dq_out_stride, l.dk_out_stride};
    const int32_t hd6[6] = {hq, hkv, hq, hkv, hq, hkv};
    for (int i = 0; i < 6; ++i)
        if ((st = check_stride(st6[i], hd6[i], head_dim, dtype)) != QKNR_OK)
            return st;
    if (o.grouped() && group_tpi(hq, hkv, head_dim, rotary_dim, dtype, true,
                                 (o.flags & QKNR_FLAG_HEAD_WEIGHTS) != 0) == 0)
        return QKNR_ERR_UNSUPPORTED;
    const size_t need = bwd_workspace_bytes_opt(tokens, hq, hkv, head_dim, rotary_dim, dtype, o);
    if (!workspace || workspace_bytes < need)
        return QKNR_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return QKNR_ERR_MISALIGNED;
    const Plan pl = make_plan(tokens, hq, hkv, head_dim, rotary_dim, dtype);
    Params p;
    fill_params(p, pl, q, k, wq, wk, pos, tokens, hq, hkv, head_dim, rotary_dim, eps, theta, o);
    // The backward reads no bias; has_b asks for the bias gradients.
    p.b[0] = p.b[1] = nullptr;
    p.has_b = gr.dbq ? 1 : 0;
    p.dy[0] = dq_out;
    p.dy[1] = dk_out;
    p.out[0] = dq;
    p.out[1] = dk;
    p.partials = static_cast<float *>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool il = (o.flags & QKNR_FLAG_INTERLEAVED) != 0;
    if (o.grouped()) {
        const bool head_w = p.head_w != 0;
        const int nq = head_w ? hq * head_dim : head_dim, nk = head_w ? hkv * head_dim : head_dim;
        const GradCols gc = {{p.has_w ? gr.dwq : nullptr, p.has_w ? gr.dwk : nullptr,
                              p.has_b ? gr.dbq : nullptr, p.has_b ? gr.dbk : nullptr},
                             {nq, nk}};
        const GwaveShape sh = gwave_shape(hq, hkv, head_dim, dtype, o.gq, o.gk);
        if (sh.tb > 0) {
            const Plan gp = gwave_plan(tokens, hq, hkv, head_dim, dtype, sh);
            p.tb_tokens = gp.tb_tokens;
            p.groups = gp.groups;
            p.token_blocks = gp.token_blocks;
            p.stages = sh.stages;
            const hipError_t e = dtype == QKNR_BF16
                                     ? gwave_dispatch<Bf16, true>(p, gp, head_dim, il, gc, s)
                                     : gwave_dispatch<float, true>(p, gp, head_dim, il, gc, s);
            return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
        }
        p.tb_tokens = group_tpi(hq, hkv, head_dim, rotary_dim, dtype, true, head_w);
        const int64_t maxb = group_blocks(tokens, p.tb_tokens);
        const hipError_t e = dtype == QKNR_BF16
                                 ? group_dispatch<Bf16, true>(p, head_dim, il, maxb, gc, s)
                                 : group_dispatch<float, true>(p, head_dim, il, maxb, gc, s);
        return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
    }
    const bool ext = p.layernorm || p.has_b;
    hipError_t e;
    if (dtype == QKNR_BF16)
        e = ext ? bwd_dispatch<Bf16, true>(p, pl, head_dim, il, gr, s)
                : bwd_dispatch<Bf16, false>(p, pl, head_dim, il, gr, s);
    else
        e = ext ? bwd_dispatch<float, true>(p, pl, head_dim, il, gr, s)
                : bwd_dispatch<float, false>(p, pl, head_dim, il, gr, s);
    return e == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

int bfd_npow2(int32_t n)
{
    int p = 1;
    while (p < n)
        p <<= 1;
    return p;
}

// Workspace layout: keys (8-byte, npow2), then rank [n], fill, ndoc, first
// [max_bins] (4-byte each), every part 16-byte aligned.
size_t bfd_workspace_bytes(int32_t ndocs, int32_t max_bins)
{
    auto up = [](size_t b) { return (b + 15) & ~(size_t)15; };
    return up(8 * (size_t)bfd_npow2(ndocs)) + up(4 * (size_t)(ndocs > 0 ? ndocs : 1)) +
           3 * up(4 * (size_t)max_bins);
}

constexpr int32_t kBfdMaxDocs = 1 << 22;

// ---- the backward that allocates nothing ----------------------------------------
//
// qknr_bwd_noalloc keeps the backward's per-workgroup weight-gradient partials
// in this file-scope device array instead of a caller workspace.  The plain
// backward needs at most kMaxBwdBlocks partial rows of 4 head_dim fp32 values
// (head_dim <= 256): 2 MiB, so every supported size fits.  Each GPU holds its
// own copy of the array until the process ends; every call on a GPU shares it
// (the partials need no clearing: each call writes every row it reads), so
// calls that overlap on one GPU race.
constexpr size_t kScratchBytes = (size_t)kMaxBwdBlocks * 4 * kMaxHeadDim * sizeof(float);
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// The device address of `scratch` on the current device, looked up once per
// device with that device current (the array's name is only a host-side
// stand-in for it) and kept.
struct ScratchAddresses {
    std::mutex m;
    void *ptr[kMaxDevices] = {};
};

qknr_status scratch_address(void **out)
{
    static ScratchAddresses cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QKNR_ERR_HIP;
    std::lock_guard<std::mutex> g(cache.m);
    if (!cache.ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return QKNR_ERR_HIP;
        cache.ptr[dev] = p;
    }
    *out = cache.ptr[dev];
    return QKNR_OK;
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
    return run_fwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, make_options(0u, nullptr, hq, hkv, head_dim), q_out, k_out, stream);
}

qknr_status qknr_fwd_ex(const void *q, const void *k, const void *wq, const void *wk,
                        const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                        int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                        qknr_dtype dtype, uint32_t flags, const qknr_layout *layout,
                        void *q_out, void *k_out, void *stream)
{
    return run_fwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, make_options(flags, layout, hq, hkv, head_dim), q_out, k_out, stream);
}

size_t qknr_bwd_workspace_bytes(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                                qknr_dtype dtype)
{
    return bwd_workspace_bytes(tokens, hq, hkv, head_dim, dtype);
}

qknr_status qknr_bwd(const void *q, const void *k, const void *wq, const void *wk,
                     const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                     int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                     qknr_dtype dtype, const void *dq_out, const void *dk_out, void *dq,
                     void *dk, void *dwq, void *dwk, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    const Grads gr = {dwq, dwk, nullptr, nullptr};
    return run_bwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, make_options(0u, nullptr, hq, hkv, head_dim), dq_out, dk_out, dq, dk,
                   gr, workspace, workspace_bytes, stream);
}

qknr_status qknr_bwd_ex(const void *q, const void *k, const void *wq, const void *wk,
                        const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                        int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                        qknr_dtype dtype, uint32_t flags, const qknr_layout *layout,
                        const void *dq_out, const void *dk_out, void *dq, void *dk, void *dwq,
                        void *dwk, void *workspace, size_t workspace_bytes, void *stream)
{
    const Grads gr = {dwq, dwk, nullptr, nullptr};
    return run_bwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, make_options(flags, layout, hq, hkv, head_dim), dq_out, dk_out, dq, dk,
                   gr, workspace, workspace_bytes, stream);
}

qknr_status qknr_bwd_noalloc(const void *q, const void *k, const void *wq, const void *wk,
                             const int32_t *position_ids, int64_t tokens, int32_t hq,
                             int32_t hkv, int32_t head_dim, int32_t rotary_dim, float eps,
                             double theta, qknr_dtype dtype, const void *dq_out,
                             const void *dk_out, void *dq, void *dk, void *dwq, void *dwk,
                             void *stream)
{
    if (bwd_workspace_bytes(tokens, hq, hkv, head_dim, dtype) > kScratchBytes)
        return QKNR_ERR_WORKSPACE;
    void *ws = nullptr;
    if (tokens > 0) {
        const qknr_status st = scratch_address(&ws);
        if (st != QKNR_OK)
            return st;
    }
    const Grads gr = {dwq, dwk, nullptr, nullptr};
    return run_bwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, make_options(0u, nullptr, hq, hkv, head_dim), dq_out, dk_out, dq, dk,
                   gr, ws, kScratchBytes, stream);
}

size_t qknr_bwd_opt_workspace_bytes(int64_t tokens, int32_t hq, int32_t hkv, int32_t head_dim,
                                    int32_t rotary_dim, qknr_dtype dtype,
                                    const qknr_options *options)
{
    if (check_shape(head_dim, rotary_dim, dtype) != QKNR_OK || hq < 1 || hkv < 1)
        return 0;
    Options o;
    if (options_from(options, hq, hkv, head_dim, rotary_dim, &o) != QKNR_OK)
        return 0;
    return bwd_workspace_bytes_opt(tokens, hq, hkv, head_dim, rotary_dim, dtype, o);
}

qknr_status qknr_fwd_opt(const void *q, const void *k, const void *wq, const void *wk,
                         const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                         qknr_dtype dtype, const qknr_options *options, void *q_out, void *k_out,
                         void *stream)
{
    qknr_status st = check_shape(head_dim, rotary_dim, dtype);
    if (st != QKNR_OK)
        return st;
    Options o;
    st = options_from(options, hq, hkv, head_dim, rotary_dim, &o);
    if (st != QKNR_OK)
        return st;
    return run_fwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, o, q_out, k_out, stream);
}

qknr_status qknr_bwd_opt(const void *q, const void *k, const void *wq, const void *wk,
                         const int32_t *position_ids, int64_t tokens, int32_t hq, int32_t hkv,
                         int32_t head_dim, int32_t rotary_dim, float eps, double theta,
                         qknr_dtype dtype, const qknr_options *options, const void *dq_out,
                         const void *dk_out, void *dq, void *dk, void *dwq, void *dwk, void *dbq,
                         void *dbk, void *workspace, size_t workspace_bytes, void *stream)
{
    qknr_status st = check_shape(head_dim, rotary_dim, dtype);
    if (st != QKNR_OK)
        return st;
    Options o;
    st = options_from(options, hq, hkv, head_dim, rotary_dim, &o);
    if (st != QKNR_OK)
        return st;
    const Grads gr = {dwq, dwk, dbq, dbk};
    return run_bwd(q, k, wq, wk, position_ids, tokens, hq, hkv, head_dim, rotary_dim, eps, theta,
                   dtype, o, dq_out, dk_out, dq, dk, gr, workspace, workspace_bytes, stream);
}

size_t qknr_bfd_workspace_bytes(int32_t ndocs, int32_t max_bins)
{
    if (ndocs < 0 || ndocs > kBfdMaxDocs || max_bins < 1 || max_bins > kBfdMaxBins)
        return 0;
    return bfd_workspace_bytes(ndocs, max_bins);
}

qknr_status qknr_bfd_pack(const int32_t *lengths, int32_t ndocs, int32_t capacity,
                          int32_t max_bins, int32_t *doc_start, int32_t *position_ids,
                          int32_t *cu_seqlens, int32_t *counts, int32_t *status, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    if (ndocs < 0 || ndocs > kBfdMaxDocs || capacity < 1 || max_bins < 1 ||
        max_bins > kBfdMaxBins || (int64_t)max_bins * capacity > INT32_MAX)
        return QKNR_ERR_INVALID_ARG;
    if ((ndocs > 0 && (!lengths || !doc_start)) || !position_ids || !cu_seqlens || !counts ||
        !status)
        return QKNR_ERR_INVALID_ARG;
    const void *ptrs[6] = {lengths, doc_start, position_ids, cu_seqlens, counts, status};
    for (const void *q : ptrs)
        if (q && !aligned(q, 4))
            return QKNR_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < bfd_workspace_bytes(ndocs, max_bins))
        return QKNR_ERR_WORKSPACE;
    if (!aligned(workspace, 16))
        return QKNR_ERR_MISALIGNED;
    const int npow2 = bfd_npow2(ndocs);
    auto up = [](size_t b) { return (b + 15) & ~(size_t)15; };
    char *ws = static_cast<char *>(workspace);
    BfdWork w;
    w.keys = reinterpret_cast<uint64_t *>(ws);
    ws += up(8 * (size_t)npow2);
    w.rank = reinterpret_cast<int32_t *>(ws);
    ws += up(4 * (size_t)(ndocs > 0 ? ndocs : 1));
    w.fill = reinterpret_cast<int32_t *>(ws);
    ws += up(4 * (size_t)max_bins);
    w.ndoc = reinterpret_cast<int32_t *>(ws);
    ws += up(4 * (size_t)max_bins);
    w.first = reinterpret_cast<int32_t *>(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // up to 64 bins: one wave with the bins in registers; more: the whole
    // workgroup, 1, 2 or 4 bins per thread (capacities of 2^20 and more take
    // the single-wave LDS loop)
    auto place = max_bins <= 64     ? qknr_bfd_place_kernel<1, 0>
                 : max_bins <= 1024 ? qknr_bfd_place_kernel<0, 1>
                 : max_bins <= 2048 ? qknr_bfd_place_kernel<0, 2>
                                    : qknr_bfd_place_kernel<0, 4>;
    hipLaunchKernelGGL(place, dim3(1), dim3(kBfdThreads), 0, s, lengths, ndocs, npow2, capacity,
                       max_bins, w, doc_start, cu_seqlens, counts, status);
    if (hipGetLastError() != hipSuccess)
        return QKNR_ERR_HIP;
    hipLaunchKernelGGL(qknr_bfd_emit_kernel, dim3((unsigned)(ndocs + max_bins)), dim3(256), 0, s,
                       lengths, ndocs, capacity, w, (const int32_t *)doc_start, position_ids,
                       cu_seqlens, (const int32_t *)counts, (const int32_t *)status);
    return hipGetLastError() == hipSuccess ? QKNR_OK : QKNR_ERR_HIP;
}

}  // extern "C"
