// Backward pass for bfloat16 storage on gfx950: the query side on the matrix cores, the key side
// with packed dot products, both streaming shifted row blocks through LDS.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv
// 2606.28560): §2 "Attended set" (window distances 0..W plus one slot per rung at d = alpha f,
// read by linear interpolation between rows i - floor(d) and i - floor(d) - 1, RoPE before the
// gather) and §2 "Per-layer scalar" (alpha = 0.5 + sigmoid(theta): the interpolation weight t is
// what carries a gradient to alpha). Gradients are of sum(do * o).
//
// Inputs come from prep_kv16 (the layout the forward reads too): rotated keys and values with dims
// permuted (element 4m + c of a row holds dim 16c + m), fp16, plus the cos/sin table. Contractions
// over dims (scores, dP) read them against q and do permuted the same way.
//
//  * bwd_q_mfma: workgroup = (batch, kv head, 4 query heads, 64 positions), lanes as in the forward
//    (fibattn_mfma.h). Two passes over the staged blocks (the near block, rows i0 - 64 .. i0 + 63,
//    for the window and the rungs with floor(d) <= 63, then far steps of two larger rungs):
//      AB, keys and values staged together: scores s (base 2), recomputed in fp32 from fp16
//         operands, dP = do . value row, and for every rung far - near of both products; then in
//         registers p = softmax(s), delta = sum p dP, dS = p (dP - delta), and the d(loss)/dt
//         terms dS (q . (k_far - k_near)) / sqrt(D) + p do . (v_far - v_near);
//      C, keys again: dq_rot = sum dS/sqrt(D) (coefficient) key row, with transposing reads of the
//         permuted keys (a lane then holds 16 consecutive dims of 4 heads), RoPE transposed
//         between lanes x and x ^ 2, written as dq.
//    It also writes, for the key side, the rotated queries and do (fp16, dims permuted) and per
//    query the (p, dS/sqrt(D)) fp16 pair of every window distance and of every rung (without the
//    rung's coefficients, which the key side applies).
//  * bwd_k_dot: workgroup = (batch, kv head, 64 key rows). Key row j is read by query j + delta of
//    every term (window distance d; the near row of a rung at a, coefficient 1 - t; its far row at
//    a + 1, coefficient t). For each query head, the near block of rotated queries and do (query
//    rows j0 .. j0 + 127: the window and the rungs with floor(d) <= 63) and then far steps of two
//    larger rungs are staged; the window runs on v_mfma_f32_16x16x16f16 as a banded product, the
//    rung terms accumulate dk_rot[j] += w_dS q_rot, dv[j] += w_p do 4 terms at a time from
//    transposing reads (a lane gets 4 rows' element of one block) with two v_dot2 per element.
//  * dalpha (fibattn_bwd.hip): fixed-order sum of the per-workgroup dt partials.
// q and do arrive by non-temporal DMA (read once) and dq, dk, dv leave by non-temporal stores; the
// rows and weights the query side writes for the key side keep plain stores, since the key side
// reads them right after (hinting them cost the key side more than it saved).
// No atomics: results are bitwise reproducible.
#include <algorithm>
#include <atomic>

#include "fibattn_mfma.h"

namespace fibattn {

namespace {

using namespace mx;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

// fp16 p in the low half, fp16 ds in the high half (bf16 p loses too much of dv: 2^-9 per term)
__device__ __forceinline__ uint32_t pack_p_ds(float p, float ds) { return pack_h2(p, ds); }

// Power-of-two scaling. fp16 holds a row exactly enough only near the unit scale, so q, do and
// the score gradients are kept as row / 2^e, e the exponent of the row's largest element (its
// floor(log2), clamped to [-126, 126]: then 2^-e is a normal float): the scaled row's largest
// element lies in [1, 2), whatever the magnitude of the inputs. Products of scaled rows are scaled
// back exactly in float32. An all-zero row has no exponent (kNoExp) and is kept as it is.
constexpr int kNoExp = -1000;
constexpr int kExpBias = 128;                          // exponents stored in bytes of the exps word

__device__ __forceinline__ int floor_log2(float x) {   // x >= 0
    if (!(x > 0.f)) return kNoExp;
    return min(max(__builtin_amdgcn_frexp_expf(x) - 1, -126), 126);
}
__device__ __forceinline__ float pow2f(int e) { return __builtin_amdgcn_ldexpf(1.0f, e); }
// A query tile's exponents for the key side, one word per (batch, head, tile): q scaled by 2^-tq,
// do by 2^-td, dS/sqrt(D) by 2^-ts (bytes 0, 1, 2, each biased by kExpBias; clamped to a byte).
__device__ __forceinline__ uint32_t pack_exps(int tq, int td, int ts) {
    auto byte = [](int e) { return static_cast<uint32_t>(min(max(e, -127), 127) + kExpBias); };
    return byte(tq) | (byte(td) << 8) | (byte(ts) << 16);
}
__device__ __forceinline__ int exps_tq(uint32_t w) { return static_cast<int>(w & 0xffu) - kExpBias; }
__device__ __forceinline__ int exps_td(uint32_t w) { return static_cast<int>((w >> 8) & 0xffu) - kExpBias; }
__device__ __forceinline__ int exps_ts(uint32_t w) { return static_cast<int>((w >> 16) & 0xffu) - kExpBias; }
// query heads per key-value head the key side takes (its factor table)
constexpr int kMaxGKey = 8;
// an h2 whose halves are 2^e (0 below fp16's subnormals)
__device__ __forceinline__ uint32_t pow2_h2(int e_lo, int e_hi) {
    return pack_h2(e_lo < -30 ? 0.f : pow2f(e_lo), e_hi < -30 ? 0.f : pow2f(e_hi));
}
__device__ __forceinline__ uint32_t mul_h2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2_t, a) * __builtin_bit_cast(h2_t, b));
}
// floor(log2) of a largest magnitude given as bf16 bits (kNoExp for 0), clamped as floor_log2
__device__ __forceinline__ int floor_log2_bits(uint32_t m) {
    if (m == 0u) return kNoExp;
    return min(max(static_cast<int>(m >> 7) - 127, -126), 126);
}
// A row's scaling exponent where fp16 holds rows with a largest magnitude in [2^-10, 2^15) well as
// they are: 0 there, else floor(log2) (the row scaled into [1, 2)); kNoExp stays.
__device__ __forceinline__ int banded(int e) { return (e >= -10 && e <= 14) ? 0 : e; }
// whether pred holds on some lane of the wave (uniform)
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }
// the largest of v over the 16 lanes of a wave with the same quad lane x (one head's positions)
__device__ __forceinline__ int head_max(int v) {
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) v = max(v, __shfl_xor(v, off, 64));
    return v;
}

// ------------------------------------------------------------------------------------------------
// The float32 tiles of the backward: for tiles that read staged key or value rows outside fp16's
// range. A query tile so flagged leaves its outputs to its float32 tile, and marks its exps word;
// every key tile that reads from a marked query tile computes its outputs in float32 too. Both are
// computed from the caller's bf16 rows and the cos/sin table: thread 8p' + e takes dims
// 8e .. 8e + 7 of a row (32 rows at a time). Slot sl of query i: sl < 16 is window distance sl,
// 16 + n kept rung n. Rows come straight from global memory: slow, and only for such tiles.
// ------------------------------------------------------------------------------------------------
constexpr int kFbSlots = 32;
constexpr uint32_t kExpsFallback = 1u << 24;         // exps word of a query tile left to the float32 tiles

__device__ __forceinline__ void load_eighth(const bf16_t* row, int e, float (&out)[8]) {
    const uint4 w = reinterpret_cast<const uint4*>(row)[e];
    const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        out[2 * h] = bf16_lo(v[h]);
        out[2 * h + 1] = bf16_hi(v[h]);
    }
}

struct FbRows {                                        // one unit's key and value rows
    const bf16_t* k;
    const bf16_t* v;
    const float* cstab;
    int e;
    // x . (rotated key row j), or (value row j), over the 64 dims of the group
    __device__ __forceinline__ float dot_k(const float (&x)[8], int j) const {
        float r[8];
        rot_eighth(k + static_cast<int64_t>(j) * kD, cstab, j, e, r);
        float d = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) d = fmaf(x[u], r[u], d);
        return oct_sum(d);
    }
    __device__ __forceinline__ float dot_v(const float (&x)[8], int j) const {
        float r[8];
        load_eighth(v + static_cast<int64_t>(j) * kD, e, r);
        float d = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) d = fmaf(x[u], r[u], d);
        return oct_sum(d);
    }
};

// Slot sl of query i: rows j (weight 1 - t) and j - 1 (weight t), or j = -1 (not attended).
__device__ __forceinline__ void fb_slot_rows(const BwdArgs& A, int sl, int i, int& j, float& t) {
    t = 0.f;
    j = -1;
    if (sl < 16) {
        if (sl <= A.W && i >= sl) j = i - sl;
    } else if (sl - 16 < A.n_off) {
        const int n = sl - 16;
        if (i >= A.off[n].a + A.off[n].interp) {
            j = i - A.off[n].a;
            t = A.off[n].interp ? A.off[n].t : 0.f;
        }
    }
}

// Softmax statistics of query i (rotated q, do in the lane's 8 dims): the largest score m (base 2),
// l = sum 2^(s - m), delta = sum p dP; and slot sl0's score and dP.
__device__ __forceinline__ void fb_query_stats(const BwdArgs& A, const FbRows& R, int i, const float (&qv)[8],
                                               const float (&dov)[8], int sl0, float& m, float& l, float& delta,
                                               float& s0, float& dp0) {
    constexpr float kNegInf = -__builtin_huge_valf();
    m = kNegInf;
#pragma unroll 1
    for (int sl = 0; sl < kFbSlots; ++sl) {
        int j;
        float t;
        fb_slot_rows(A, sl, i, j, t);
        if (j < 0) continue;
        float sc = R.dot_k(qv, j);
        if (t != 0.f) sc = fmaf(t, R.dot_k(qv, j - 1) - sc, sc);
        m = fmaxf(m, sc * A.qscale);
    }
    l = 0.f;
    float dsum = 0.f;
    s0 = kNegInf;
    dp0 = 0.f;
#pragma unroll 1
    for (int sl = 0; sl < kFbSlots; ++sl) {
        int j;
        float t;
        fb_slot_rows(A, sl, i, j, t);
        if (j < 0) continue;
        float sc = R.dot_k(qv, j), dpv = R.dot_v(dov, j);
        if (t != 0.f) {
            sc = fmaf(t, R.dot_k(qv, j - 1) - sc, sc);
            dpv = fmaf(t, R.dot_v(dov, j - 1) - dpv, dpv);
        }
        sc *= A.qscale;
        const float ex = __builtin_amdgcn_exp2f(sc - m);
        l += ex;
        dsum = fmaf(ex, dpv, dsum);
        if (sl == sl0) {
            s0 = sc;
            dp0 = dpv;
        }
    }
    delta = dsum / l;
}

// dq and the d(loss)/dt partials of one query tile (the workgroup's), in float32.
__device__ __forceinline__ void bwd_q_tile_fp32(const BwdArgs& A, int b, int bg, int h0, int i0, int slot, char* lds) {
    float* dtbuf = reinterpret_cast<float*>(lds);                  // [64][16] d(loss)/dt per rung
    const int e = threadIdx.x & 7, gi = threadIdx.x >> 3, L = A.L;
    const FbRows R{static_cast<const bf16_t*>(A.k) + static_cast<int64_t>(bg) * L * kD,
                   static_cast<const bf16_t*>(A.v) + static_cast<int64_t>(bg) * L * kD, A.cstab, e};
    float dt_sum = 0.f;                                             // thread n < 16: rung n's partial
#pragma unroll 1
    for (int hh = 0; hh < 4; ++hh) {
        for (int u = threadIdx.x; u < kTile * 16; u += kNT) dtbuf[u] = 0.f;
        __syncthreads();
        const int h = h0 + hh;
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
            const int pp = 32 * half + gi, i = i0 + pp;
            if (i >= L) continue;                                   // whole groups skip together
            const int64_t qrow = (static_cast<int64_t>(b) * A.Hq + h) * L + i;
            float qv[8], dov[8];
            rot_eighth(static_cast<const bf16_t*>(A.q) + qrow * kD, A.cstab, i, e, qv);
            load_eighth(static_cast<const bf16_t*>(A.dout) + qrow * kD, e, dov);
            float m, l, delta, s0, dp0;
            fb_query_stats(A, R, i, qv, dov, -1, m, l, delta, s0, dp0);
            float dq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int sl = 0; sl < kFbSlots; ++sl) {
                int j;
                float t;
                fb_slot_rows(A, sl, i, j, t);
                if (j < 0) continue;
                float kn[8];
                rot_eighth(R.k + static_cast<int64_t>(j) * kD, A.cstab, j, e, kn);
                float sc = 0.f, dpv = R.dot_v(dov, j);
                {
                    float d = 0.f;
#pragma unroll
                    for (int u = 0; u < 8; ++u) d = fmaf(qv[u], kn[u], d);
                    sc = oct_sum(d);
                }
                float gk = 0.f, gv = 0.f;
                if (t != 0.f) {
                    float kf[8];
                    rot_eighth(R.k + static_cast<int64_t>(j - 1) * kD, A.cstab, j - 1, e, kf);
                    float d = 0.f;
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        d = fmaf(qv[u], kf[u], d);
                        kn[u] = fmaf(t, kf[u] - kn[u], kn[u]);     // the blended key row
                    }
                    const float sf = oct_sum(d), dvf = R.dot_v(dov, j - 1);
                    gk = sf - sc;                                   // q . (k_far - k_near)
                    gv = dvf - dpv;                                 // do . (v_far - v_near)
                    sc = fmaf(t, gk, sc);
                    dpv = fmaf(t, gv, dpv);
                }
                const float pr = __builtin_amdgcn_exp2f(sc * A.qscale - m) / l;
                const float ds = pr * (dpv - delta) * A.scale;     // dS / sqrt(D)
#pragma unroll
                for (int u = 0; u < 8; ++u) dq[u] = fmaf(ds, kn[u], dq[u]);
                if (sl >= 16 && t != 0.f && e == 0) dtbuf[pp * 16 + (sl - 16)] = fmaf(ds, gk, pr * gv);
            }
            // dq = RoPE transposed at i: x = x' c + y' s (dims below 32), y = y' c - x' s; the pair's
            // other half is in lane e ^ 4 of the group
            const float4* cs = reinterpret_cast<const float4*>(A.cstab + static_cast<int64_t>(i) * 2 * kPairs + 16 * (e & 3));
            const float sg = (e < 4) ? 1.f : -1.f;
            float out[8];
#pragma unroll
            for (int hp = 0; hp < 4; ++hp) {
                const float4 t = cs[hp];
                const float o0 = __shfl_xor(dq[2 * hp], 4, 64), o1 = __shfl_xor(dq[2 * hp + 1], 4, 64);
                out[2 * hp] = fmaf(sg * o0, t.y, dq[2 * hp] * t.x);
                out[2 * hp + 1] = fmaf(sg * o1, t.w, dq[2 * hp + 1] * t.z);
            }
            store_nt(static_cast<bf16_t*>(A.dq) + qrow * kD + 8 * e,
                     make_uint4(pack_bf2(out[0], out[1]), pack_bf2(out[2], out[3]), pack_bf2(out[4], out[5]),
                                pack_bf2(out[6], out[7])));
        }
        __syncthreads();                                            // dtbuf is complete
        if (threadIdx.x < 16) {
            for (int pp = 0; pp < kTile; ++pp)
                if (i0 + pp < L) dt_sum += dtbuf[pp * 16 + threadIdx.x];
        }
        __syncthreads();                                            // before the next head's buffer
    }
    if (threadIdx.x < static_cast<unsigned>(A.n_off))
        A.partial[static_cast<int64_t>(slot) * kMaxOff + threadIdx.x] = threadIdx.x < 16 ? dt_sum : 0.f;
}

// dk and dv of one key tile (rows j0 .. j0 + 63 of unit bg, key-value head g), in float32: key row j
// is read by query j + d of window distance d, by query j + a (weight 1 - t, or 1 if integral) as
// the nearer row of rung a and by query j + a + 1 (weight t) as the farther one; each such term
// recomputes its query's softmax statistics.
__device__ __forceinline__ void bwd_k_tile_fp32(const BwdArgs& A, int b, int bg, int g, int j0) {
    const int e = threadIdx.x & 7, gi = threadIdx.x >> 3, L = A.L;
    const FbRows R{static_cast<const bf16_t*>(A.k) + static_cast<int64_t>(bg) * L * kD,
                   static_cast<const bf16_t*>(A.v) + static_cast<int64_t>(bg) * L * kD, A.cstab, e};
    const int n_terms = 16 + 2 * A.n_off;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
        const int j = j0 + 32 * half + gi;
        if (j >= L) continue;
        float dk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, dv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int hh = 0; hh < A.G; ++hh) {
            const int h = g * A.G + hh;
#pragma unroll 1
            for (int tm = 0; tm < n_terms; ++tm) {
                // term tm: window distance tm (< 16), or rung n = (tm - 16) / 2 as nearer / farther row
                int i, sl;
                float coef = 1.f;
                if (tm < 16) {
                    if (tm > A.W) continue;
                    i = j + tm;
                    sl = tm;
                } else {
                    const int n = (tm - 16) >> 1, far = (tm - 16) & 1;
                    const int a = A.off[n].a, ip = A.off[n].interp;
                    const float t = A.off[n].t;
                    if (far && !ip) continue;
                    i = j + a + far;
                    if (i < a + ip) continue;                       // the query does not attend this rung
                    sl = 16 + n;
                    coef = ip ? (far ? t : 1.f - t) : 1.f;
                }
                if (i >= L) continue;
                const int64_t qrow = (static_cast<int64_t>(b) * A.Hq + h) * L + i;
                float qv[8], dov[8];
                rot_eighth(static_cast<const bf16_t*>(A.q) + qrow * kD, A.cstab, i, e, qv);
                load_eighth(static_cast<const bf16_t*>(A.dout) + qrow * kD, e, dov);
                float m, l, delta, s0, dp0;
                fb_query_stats(A, R, i, qv, dov, sl, m, l, delta, s0, dp0);
                const float pr = __builtin_amdgcn_exp2f(s0 - m) / l;
                const float ds = pr * (dp0 - delta) * A.scale;     // dS / sqrt(D)
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    dk[u] = fmaf(coef * ds, qv[u], dk[u]);
                    dv[u] = fmaf(coef * pr, dov[u], dv[u]);
                }
            }
        }
        // dk = RoPE transposed at j (the pair's other half in lane e ^ 4)
        const float4* cs = reinterpret_cast<const float4*>(A.cstab + static_cast<int64_t>(j) * 2 * kPairs + 16 * (e & 3));
        const float sg = (e < 4) ? 1.f : -1.f;
        float out[8];
#pragma unroll
        for (int hp = 0; hp < 4; ++hp) {
            const float4 t = cs[hp];
            const float o0 = __shfl_xor(dk[2 * hp], 4, 64), o1 = __shfl_xor(dk[2 * hp + 1], 4, 64);
            out[2 * hp] = fmaf(sg * o0, t.y, dk[2 * hp] * t.x);
            out[2 * hp + 1] = fmaf(sg * o1, t.w, dk[2 * hp + 1] * t.z);
        }
        const int64_t krow = (static_cast<int64_t>(bg) * L + j) * kD + 8 * e;
        store_nt(static_cast<bf16_t*>(A.dk) + krow, make_uint4(pack_bf2(out[0], out[1]), pack_bf2(out[2], out[3]),
                                                                 pack_bf2(out[4], out[5]), pack_bf2(out[6], out[7])));
        store_nt(static_cast<bf16_t*>(A.dv) + krow, make_uint4(pack_bf2(dv[0], dv[1]), pack_bf2(dv[2], dv[3]),
                                                                 pack_bf2(dv[4], dv[5]), pack_bf2(dv[6], dv[7])));
    }
}

// ------------------------------------------------------------------------------------------------
// bwd_q_mfma
// ------------------------------------------------------------------------------------------------
// PRECISE: scores from split operands (q and the staged keys each as a high and a low fp16 part),
// for calls that ask for d(alpha): that one scalar sums every (query, head, rung) term with heavy
// cancellation and would otherwise inherit the 2^-11 rounding of q and k relative to its
// (small) value. Pass AB then runs as pass A (keys and their low parts: scores) and pass B
// (values: dP).
// INT: every kept rung is integral (the integer-offset path of §2 "Implementation note"; d(alpha)
// is not defined there, so never with PRECISE): as in the forward, the rungs with a <= 64 come from
// the near block four to a group (at most two groups) and far steps stage 64-row blocks of the
// near rows alone. The hand-off to the key side stays indexed by rung.
template <int MAXS, bool PRECISE, bool INT>
__global__ __launch_bounds__(kNT, 2) void bwd_q_mfma_kernel(BwdArgs A) {
    static_assert(!(PRECISE && INT), "d(alpha) is not defined for integral rungs");
    constexpr int MAXK = 2 * MAXS;
    // Two item buffers used in turn, each a key part and a value part. Items: the key and value
    // near blocks, then the key and value far steps (pass AB); then the key near block and key
    // far steps again (pass C, key parts only).
    __shared__ __attribute__((aligned(1024))) char lds0[2 * kBufBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[2 * kBufBytes];
    __shared__ float red[4][MAXK];
    __shared__ int ered[4][4][3];                       // [wave][head]: largest exponents of q, do, dS
    __shared__ int votes[4];                            // per wave: a staged row it checks lies outside fp16's range

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int pq = lane >> 2, x = lane & 3;
    const int p = 16 * wave + pq;
    const int L = A.L, W = A.W;
    const int n_tiles = (L + kTile - 1) / kTile;
    const int n_chunk = A.G >> 2;
    int unit, tile;
    unit_tile(blockIdx.x, n_tiles, A.xcd_map, unit, tile);
    const int chunk = unit % n_chunk;
    const int bg = unit / n_chunk;
    const int b = bg / A.Hkv;
    const int h0 = (bg % A.Hkv) * A.G + chunk * 4;
    const int i0 = tile * kTile;
    const int i = i0 + p;
    const bool active = i < L;

    // (counted over the packed scan table, RungScan: a few wide scalar loads, where a loop over
    // the offset table waits for each rung's load in turn)
    int n_reach = 0, n_lo = 0;
#pragma unroll
    for (int n = 0; n < kScanRungs; ++n) {
        n_reach += (A.scan.r[n] <= i0 + kTile - 1) ? 1 : 0;
        n_lo += (A.scan.a[n] <= kNear - (INT ? 0 : 1)) ? 1 : 0;
    }
    // near rungs: the prefix with a <= 63 (near and far rows inside the near block, key rows
    // i0 - 64 .. i0 + 63; INT: a <= 64, the one row). Steps k < kn come from the near block, kn
    // even: rung pairs 2k, 2k + 1, or (INT) for even k a group of the four rungs 2k .. 2k + 3
    // (those past nn are padding). Steps kn .. n_steps - 1 are far steps, step k in buffer
    // (k + 1) % 2, holding rungs 2k - ro and 2k - ro + 1 (ro = 0 unless INT). Products of step k
    // go to slots 2k and 2k + 1 (a near group: 2k .. 2k + 3).
    const int n_near = min(n_lo, n_reach);
    const int nn = INT ? min(n_near, 8) : 0;
    const int kn = INT ? 2 * ((nn + 3) >> 2) : (n_near >> 1) & ~1;
    const int ro = INT ? 2 * kn - nn : 0;
    const int n_steps = INT ? kn + ((n_reach - nn + 1) >> 1) : (n_reach + 1) >> 1;
    constexpr int kStepDmas = INT ? 4 : 6;              // DMA instructions per wave of a far step

    const int64_t kv_row0 = static_cast<int64_t>(bg) * L;
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(A.kstage, kv_row0, L);
    const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(A.vstage, kv_row0, L);
    // the second half of each pass-A item: the values (fused pass AB) or the keys' low parts
    const __amdgpu_buffer_rsrc_t hrs = PRECISE ? rows_rsrc(A.kstage_lo, kv_row0, L) : vrs;
    Stager st;
    st.init(lane, wave);
    // (INT: the near row of position p at slot p or 72 + p)
    auto step = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int k) {
        if constexpr (INT) {
            const int n = 2 * k - ro;
            st.step64(rs, dst, n < n_reach, i0 - A.off[n].a, n + 1 < n_reach, i0 - A.off[n + 1].a);
        } else {
            st.step(rs, dst, 2 * k < n_reach, i0 - A.off[2 * k].a - 1, 2 * k + 1 < n_reach, i0 - A.off[2 * k + 1].a - 3);
        }
    };
    auto kv_step = [&](char* dst, int k) {         // 2 kStepDmas DMA instructions per wave
        step(krs, dst, k);
        step(hrs, dst + kBufBytes, k);
    };
    auto buf = [&](int j) -> char* { return (j & 1) ? lds1 : lds0; };
    const int jn = i0 - kNear;                          // the near block's row at slot 0

    // The 8 linear-view chunks of a wave's 8 KB region of treg to rows of a [.., L, 64] fp16 or
    // bf16 tensor (linear-view slot s is head h0 + (s >> 4) at position i0 + 16w + (s & 15)): all
    // 8 LDS reads first, then 8 buffer stores of 1 KB contiguous per instruction. A slot past L
    // stores at an offset beyond the buffer (4 heads' L rows from row (b Hq + h0) L: within 32 bits
    // for L <= 2^20), which the hardware drops, so no branch splits the reads from one another.
    // aux: 2 for non-temporal stores.
    auto store_lin = [&](void* base, const char* treg, int aux) {
        const __amdgpu_buffer_rsrc_t ors = rows_rsrc(base, (static_cast<int64_t>(b) * A.Hq + h0) * L, 4 * L);
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint4*>(treg + lin_view_addr(lane, u));
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sl = lin_slot(lane, u);
            const int pos = i0 + 16 * wave + (sl & 15);
            const int off = pos < L ? ((sl >> 4) * L + pos) * kRowBytes + (lane & 7) * 16 : -kRowBytes;
            typedef int v4i_t __attribute__((ext_vector_type(4)));
            const v4i_t d = {static_cast<int>(v[u].x), static_cast<int>(v[u].y), static_cast<int>(v[u].z), static_cast<int>(v[u].w)};
            if (aux)
                __builtin_amdgcn_raw_buffer_store_b128(d, ors, off, 0, 2);
            else
                __builtin_amdgcn_raw_buffer_store_b128(d, ors, off, 0, 0);
        }
    };

    // ---- prologue: q and do of the wave's 16 positions and 4 heads by LDS DMA into the wave's
    // 8 KB of lds0 (q) and of lds1 (do), 1 KB contiguous per instruction (lane l lands on slot
    // 8u + (l >> 3), physical chunk l & 7, and fetches the logical chunk the swizzle puts there),
    // read back one row per lane; then the key and value near blocks and far step kn ----
    uint4 qraw[8], draw[8];
    float4 ctq[4];                                      // cos/sin of pairs 8x..8x+7 at position i
    uint32_t flagged;                                   // nonzero: a staged row the lane checks lies outside fp16's range
    {
        // the 4 heads' rows (4 L rows of 128 bytes: within 32 bits for L <= 2^20); positions past
        // L read row L - 1 (finite, never used)
        const int64_t hrow = (static_cast<int64_t>(b) * A.Hq + h0) * L;
        const __amdgpu_buffer_rsrc_t qrs4 = rows_rsrc(A.q, hrow, 4 * L);
        const __amdgpu_buffer_rsrc_t drs4 = rows_rsrc(A.dout, hrow, 4 * L);
        char* const rq = lds0 + wave * 8192;
        char* const rd = lds1 + wave * 8192;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sl = lin_slot(lane, u);
            const int pos = min(i0 + 16 * wave + (sl & 15), L - 1);
            const int voff = ((sl >> 4) * L + pos) * kRowBytes + (((lane & 7) ^ tr_f(sl)) << 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs4, dma_dst(rq + u * 1024), 16, voff, 0, 0, 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(drs4, dma_dst(rd + u * 1024), 16, voff, 0, 0, 2);
        }
        const float4* ct = reinterpret_cast<const float4*>(A.cstab) + static_cast<int64_t>(active ? i : 0) * (kPairs / 2) + 4 * x;
#pragma unroll
        for (int u = 0; u < 4; ++u) ctq[u] = ct[u];
        // the range flags of the staged key and value rows this tile reads (in flight with q, do)
        flagged = rows_flagged(A, bg / kPrepRowGroup, i0, n_reach);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            qraw[c] = *reinterpret_cast<const uint4*>(rq + row_view_addr(pq, x, c));
            draw[c] = *reinterpret_cast<const uint4*>(rd + row_view_addr(pq, x, c));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();                   // every wave is done with its rows
        asm volatile("" ::: "memory");
    }
    st.near(krs, lds0, jn);
    st.near(hrs, lds0 + kBufBytes, jn);
    kv_step(lds1, kn);
    // Row exponents, behind the staging: q and do are carried as row / 2^e in fp16 (|q_rot| <=
    // sqrt(2) max|q|: one more binade of headroom). Rows fp16 holds well as they are keep e = 0,
    // except q for the scores when they must be precise (its low part needs the row near 1); q's
    // hand-off to the key side takes the banded exponent either way. Each head's largest hand-off
    // exponent over the wave's positions goes to ered; whether a staged row this tile reads lies
    // outside fp16's range is voted on (read after the next barrier).
    int eq, ed;                                         // (0 for a zero row)
    {
        const int fq = floor_log2_bits(max_abs_bf16_bits(qraw));
        const int eqh = banded(fq);
        eq = PRECISE ? fq : eqh;
        ed = banded(floor_log2_bits(max_abs_bf16_bits(draw)));
        const int mq = head_max(active ? eqh : kNoExp), md = head_max(active ? ed : kNoExp);
        if (pq == 0) {
            ered[wave][x][0] = mq;
            ered[wave][x][1] = md;
        }
        if (eq == kNoExp) eq = 0;
        if (ed == kNoExp) ed = 0;
        post_vote(votes, wave, flagged != 0u);
    }
    const bool wscaled = wave_any(eq != 0 || ed != 0);  // uniform: some row of the wave is scaled
    // head x's largest q and do exponents over the tile (read from LDS where needed: registers
    // are short here)
    auto tile_exp = [&](int k) {
        const int f = max(max(ered[0][x][k], ered[1][x][k]), max(ered[2][x][k], ered[3][x][k]));
        return f == kNoExp ? 0 : f;
    };

    // q rotated at its position (unscaled), fp16, in the keys' permuted order: word 2m holds dims
    // (m, 16 + m), word 2m + 1 dims (32 + m, 48 + m); register chunk c = words 4c..4c+3. PRECISE
    // also keeps what the fp16 rounding left out (ql, same layout).
    uint32_t q[8][4];
    uint32_t ql[PRECISE ? 8 : 1][4];
    const float qsc = A.qscale * pow2f(eq);             // the score scale of the lane's scaled row
    {
        float r[kD];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t lw[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
            const uint32_t hw[4] = {qraw[c + 4].x, qraw[c + 4].y, qraw[c + 4].z, qraw[c + 4].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 t = quad_bcast(c, ctq[m]);  // pairs 8c + 2m, 8c + 2m + 1 (from lane c)
                const float x0 = bf16_lo(lw[m]), x1 = bf16_hi(lw[m]);
                const float y0 = bf16_lo(hw[m]), y1 = bf16_hi(hw[m]);
                const int j = 8 * c + 2 * m;
                r[j] = x0 * t.x - y0 * t.y;
                r[j + 1] = x1 * t.z - y1 * t.w;
                r[j + 32] = y0 * t.x + x0 * t.y;
                r[j + 33] = y1 * t.z + x1 * t.w;
            }
        }
        if (wscaled) {
            const float sq = pow2f(-eq);
#pragma unroll
            for (int j = 0; j < kD; ++j) r[j] *= sq;
        }
#pragma unroll
        for (int w = 0; w < 32; ++w) {
            const int m = w >> 1;
            const float a0 = (w & 1) ? r[32 + m] : r[m], a1 = (w & 1) ? r[48 + m] : r[16 + m];
            q[w >> 2][w & 3] = pack_h2(a0, a1);
            if constexpr (PRECISE) {
                const h2_t hi = __builtin_bit_cast(h2_t, q[w >> 2][w & 3]);
                ql[w >> 2][w & 3] = pack_h2(a0 - static_cast<float>(hi.x), a1 - static_cast<float>(hi.y));
            }
        }
    }
    // do as fp16 in the values' permuted order (word 2m: dims (m, 16 + m), word 2m + 1: dims
    // (32 + m, 48 + m))
    uint32_t dov[8][4];
    {
        auto dim = [&](int d) -> float {               // bf16 dim d of the raw row
            const uint4& r = draw[d >> 3];
            const int w = (d >> 1) & 3;
            const uint32_t v = w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
            return (d & 1) ? bf16_hi(v) : bf16_lo(v);
        };
        if (wscaled) {
            const float sdo = pow2f(-ed);               // do / 2^ed
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                dov[m >> 1][2 * (m & 1)] = pack_h2(dim(m) * sdo, dim(16 + m) * sdo);
                dov[m >> 1][2 * (m & 1) + 1] = pack_h2(dim(32 + m) * sdo, dim(48 + m) * sdo);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                dov[m >> 1][2 * (m & 1)] = pack_h2(dim(m), dim(16 + m));
                dov[m >> 1][2 * (m & 1) + 1] = pack_h2(dim(32 + m), dim(48 + m));
            }
        }
    }
    publish<2 * kStepDmas>();                           // the key and value near blocks have landed

    // ---- pass AB: scores s (base 2) with the keys, dP = do . value row with the values, and for
    // each rung far - near of both products (PRECISE: pass A, the scores, then pass B, dP) ----
    float s[4 * kWG + MAXK], sd[MAXK], dp[4 * kWG + MAXK], dpd[MAXK];
    const int s0 = p - x + kNear;                       // window: lane x reads distance 4g + x
    const int rslot = INT ? p + ((x >> 1) ? kBlkSlots : 0)                      // far-step rung rows
                          : p + ((x >> 1) ? kBlkSlots + 2 : 0) + ((x & 1) ? 0 : 1);
    const int rbase = rslot * kRowBytes, rsw = swz(rslot);
    // a rung pair's products (lane x: rung 2k + (x >> 1), near row for x even, far row for x odd)
    auto score_terms = [&](const f4_t& acc, int k) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int n = 2 * k + e;
            if (n < n_reach) {
                const float t = A.off[n].t;
                const float dd = (acc[2 * e + 1] - acc[2 * e]) * qsc;
                const float sc = fmaf(t, dd, acc[2 * e] * qsc);
                const bool ok = active && i >= A.off[n].a + A.off[n].interp;
                s[4 * kWG + n] = ok ? sc : kNegInf;
                sd[n] = ok ? dd : 0.f;
            }
        }
    };
    // both products of a rung pair at once (one read of each rung's parameters); INT: the near
    // rows of rungs 2k - ro + e in columns 2e, slots 2k + e
    auto pair_terms = [&](const f4_t& acc, const f4_t& accv, int k) {
        if constexpr (INT) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int n = 2 * k + e - ro;
                if (n < n_reach) {
                    const bool ok = active && i >= A.off[n].a;
                    s[4 * kWG + 2 * k + e] = ok ? acc[2 * e] * qsc : kNegInf;
                    dp[4 * kWG + 2 * k + e] = accv[2 * e];
                }
            }
            return;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int n = 2 * k + e;
            if (n < n_reach) {
                const float t = A.off[n].t;
                const float dd = (acc[2 * e + 1] - acc[2 * e]) * qsc;
                const float sc = fmaf(t, dd, acc[2 * e] * qsc);
                const bool ok = active && i >= A.off[n].a + A.off[n].interp;
                s[4 * kWG + n] = ok ? sc : kNegInf;
                dp[4 * kWG + n] = fmaf(t, accv[2 * e + 1] - accv[2 * e], accv[2 * e]);
            }
        }
    };
    auto dp_terms = [&](const f4_t& accv, int k) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int n = 2 * k + e;
            if (n < n_reach) {
                const float dv = accv[2 * e + 1] - accv[2 * e];
                dp[4 * kWG + n] = fmaf(A.off[n].t, dv, accv[2 * e]);
                dpd[n] = dv;
            }
        }
    };
    // scores of one group: the row at slot byte offset base of buffer b (and its low part)
    auto qk = [&](const char* b, int base, int F) -> f4_t {
        if constexpr (PRECISE)
            return row_dot_group_x3(q, ql, b, b + kBufBytes, base, F);
        else
            return row_dot_group(q, b, base, F);
    };
    auto near_slot = [&](int k) {   // near rung pair k: near row i - a at slot p + 64 - a, far one down
        return p + kNear - pick_uniform((x >> 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a) - (x & 1);
    };
    // INT, near group of step k (even): the distance of rung 2k + c, 0 (the window's own row, a
    // staged row) for padding; lane c reads rung 2k + c at slot p + 64 - a (pass C: position pt)
    auto near_a = [&](int k, int c) -> int { return 2 * k + c < nn ? A.off[2 * k + c].a : 0; };
    auto group_a = [&](int k, int c) -> int { return pick4(c, near_a(k, 0), near_a(k, 1), near_a(k, 2), near_a(k, 3)); };
#pragma unroll
    for (int k = 0; k < MAXK; ++k) {
        s[4 * kWG + k] = kNegInf;
        sd[k] = 0.f;
        dp[4 * kWG + k] = 0.f;
        dpd[k] = 0.f;
    }
    // values in the second half of each item (fused) or in the first (pass B)
    const int voff = PRECISE ? 0 : kBufBytes;
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
        f4_t acc = {0.f, 0.f, 0.f, 0.f}, accv = {0.f, 0.f, 0.f, 0.f};
        if (4 * g <= W) {
            acc = qk(lds0, (s0 - 4 * g) * kRowBytes, swz(s0 - 4 * g));
            if constexpr (!PRECISE) accv = row_dot_group(dov, lds0 + voff, (s0 - 4 * g) * kRowBytes, swz(s0 - 4 * g));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 4 * g + r;
            s[d] = (active && d <= W && i >= d) ? acc[r] * qsc : kNegInf;
            dp[d] = accv[r];
        }
    }
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        if constexpr (INT) {
            if ((k & 1) == 0 && k < kn) {
                const int sl = p + kNear - group_a(k, x);
                const f4_t acc = qk(lds0, sl * kRowBytes, swz(sl));
                const f4_t accv = row_dot_group(dov, lds0 + voff, sl * kRowBytes, swz(sl));
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int n = 2 * k + c;
                    if (n < nn) {
                        s[4 * kWG + n] = (active && i >= A.off[n].a) ? acc[c] * qsc : kNegInf;
                        dp[4 * kWG + n] = accv[c];
                    }
                }
            }
        } else if (k < kn) {
            const int sl = near_slot(k);
            // (both products issued before either's terms: the second overlaps the first's latency)
            const f4_t acc = qk(lds0, sl * kRowBytes, swz(sl));
            if constexpr (!PRECISE) {
                pair_terms(acc, row_dot_group(dov, lds0 + voff, sl * kRowBytes, swz(sl)), k);
            } else {
                score_terms(acc, k);
            }
        }
    }
    publish<0>();                                       // far step kn has landed, buffer 0 is free
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        if (k >= kn && k < n_steps) {
            if (k + 1 < n_steps) kv_step(buf(k + 2), k + 1);
            const f4_t acc = qk(buf(k + 1), rbase, rsw);
            if constexpr (!PRECISE) {
                pair_terms(acc, row_dot_group(dov, buf(k + 1) + voff, rbase, rsw), k);
            } else {
                score_terms(acc, k);
            }
            publish<0>();
        }
    }
    if constexpr (PRECISE) {
        // ---- pass B: the values alone (near block into buffer 0, far step kn into buffer 1) ----
        st.near(vrs, lds0, jn);
        step(vrs, lds1, kn);
        publish<6>();                                   // the value near block has landed
#pragma unroll
        for (int g = 0; g < kWG; ++g) {
            f4_t accv = {0.f, 0.f, 0.f, 0.f};
            if (4 * g <= W) accv = row_dot_group(dov, lds0, (s0 - 4 * g) * kRowBytes, swz(s0 - 4 * g));
#pragma unroll
            for (int r = 0; r < 4; ++r) dp[4 * g + r] = accv[r];
        }
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if (k < kn) {
                const int sl = near_slot(k);
                dp_terms(row_dot_group(dov, lds0, sl * kRowBytes, swz(sl)), k);
            }
        }
        publish<0>();
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if (k >= kn && k < n_steps) {
                if (k + 1 < n_steps) step(vrs, buf(k + 2), k + 1);
                dp_terms(row_dot_group(dov, buf(k + 1), rbase, rsw), k);
                publish<0>();
            }
        }
    }

    // ---- key near block and key far step kn again (pass C), under the softmax ----
    st.near(krs, lds0, jn);
    step(krs, lds1, kn);
    // from here on the value halves of both buffers are free: 8 KB per wave
    char* const treg = (wave < 2 ? lds0 : lds1) + kBufBytes + (wave & 1) * 8192;
    // rotated q and do (fp16) for the key side, through treg: 1 KB contiguous stores (they count
    // in vmcnt after the key DMAs; the wait before pass C counts them conservatively). Each head's
    // rows are scaled to a common power of two over the tile, q by 2^-tq and do by 2^-td (exps
    // records tq, td for the key side)
    // whether a staged row this tile reads lies outside fp16's range (the votes, read where needed
    // rather than held): then its outputs come from the float32 tiles (its float32 tile writes dq
    // and the partials, and the key tiles that read this tile's hand-off, marked at the end,
    // compute theirs in float32 too)
    if (!or_votes(votes)) {
        const int tq = tile_exp(0), td = tile_exp(1);
        const bool tscaled = wave_any(eq != tq || ed != td);
        const uint32_t fqh = pow2_h2(eq - tq, eq - tq), fdh = pow2_h2(ed - td, ed - td);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t(&v)[4] = t ? dov[c] : q[c];
                const uint32_t f = t ? fdh : fqh;
                *reinterpret_cast<uint4*>(treg + row_view_addr(pq, x, c)) =
                    tscaled ? make_uint4(mul_h2(v[0], f), mul_h2(v[1], f), mul_h2(v[2], f), mul_h2(v[3], f))
                            : make_uint4(v[0], v[1], v[2], v[3]);
            }
            store_lin(t ? A.do16 : A.qrot16, treg, 0);
        }
    }

    float mx = kNegInf;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) mx = fmaxf(mx, s[y]);
    if (!active) mx = 0.f;
    float l = 0.f;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) {
        s[y] = __builtin_amdgcn_exp2f(s[y] - mx);
        l += s[y];
    }
    const float inv = active ? 1.0f / l : 0.f;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) s[y] *= inv;   // s now holds p

    // ---- softmax gradient ----
    float delta = 0.f;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) delta = fmaf(s[y], dp[y], delta);
    // dS = p (dP - delta) / sqrt(D), in place of dP; d(loss)/dt terms, which only a call that
    // asks for d(alpha) (PRECISE) sums: the other variants leave them out
    float dt[MAXK];
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) dp[y] = s[y] * (dp[y] - delta) * A.scale;
    if constexpr (PRECISE) {
#pragma unroll
        for (int n = 0; n < MAXK; ++n) {
            // dS (q . (k_far - k_near)) / sqrt(D) in base 2: sd = (q . dk) log2(e) / sqrt(D), so
            // (dS / sqrt(D)) sd ln2 sqrt(D) = dS (q . dk) / sqrt(D)
            dt[n] = fmaf(dp[4 * kWG + n] * (kLn2 / A.scale), sd[n], s[4 * kWG + n] * dpd[n]);
        }
        // dS/sqrt(D), dP and the dt terms are in units of 2^-ed (do was scaled by it): dt to true
        // units
        if (wscaled) {
#pragma unroll
            for (int n = 0; n < MAXK; ++n) dt[n] *= pow2f(ed);
        }
    }
    // the key side's weights of this query: (p, dS/sqrt(D)) per window distance and per rung
    // (without the rung's coefficients), fp16 pairs, dS scaled by the row's 2^-es (its largest
    // element in [1, 2)); stored at the end, once the tile's common exponent is known
    int es;
    {
        float mxd = 0.f;
#pragma unroll
        for (int y = 0; y < 4 * kWG + MAXK; ++y) mxd = fmaxf(mxd, fabsf(dp[y]));
        es = banded(floor_log2(mxd));
    }
    uint32_t wq[4 * kWG + MAXK];
    if (wave_any(es != kNoExp && es != 0)) {
        const float sds = pow2f(es == kNoExp ? 0 : -es);
#pragma unroll
        for (int y = 0; y < 4 * kWG + MAXK; ++y) wq[y] = pack_p_ds(s[y], dp[y] * sds);
    } else {
#pragma unroll
        for (int y = 0; y < 4 * kWG + MAXK; ++y) wq[y] = pack_p_ds(s[y], dp[y]);
    }
    es = (es == kNoExp || !active) ? kNoExp : es + ed;  // the row's dS exponent in true units
    // pass C weights: dS/sqrt(D) times the coefficients, fp16, groups of 4
    uint32_t ww[kWG][2], wo[MAXS][2];
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
        ww[g][0] = pack_h2(dp[4 * g], dp[4 * g + 1]);
        ww[g][1] = pack_h2(dp[4 * g + 2], dp[4 * g + 3]);
    }
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        if constexpr (INT) {
            // a near group (even k < kn): slots 2k .. 2k + 3; a far step: slots 2k, 2k + 1 in
            // group slots 0 and 2 (slots 1 and 3 weigh 0)
            auto dn = [&](int y) { return y < MAXK ? dp[4 * kWG + y] : 0.f; };
            const bool grp = k < kn && (k & 1) == 0;
            wo[k][0] = pack_h2(dn(2 * k), grp ? dn(2 * k + 1) : 0.f);
            wo[k][1] = grp ? pack_h2(dn(2 * k + 2), dn(2 * k + 3)) : pack_h2(dn(2 * k + 1), 0.f);
        } else {
            float w[4];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int n = 2 * k + e;
                const float dn = dp[4 * kWG + n];
                const float far = (n < n_reach) ? dn * A.off[n].t : 0.f;
                w[2 * e] = dn - far;
                w[2 * e + 1] = far;
            }
            wo[k][0] = pack_h2(w[0], w[1]);
            wo[k][1] = pack_h2(w[2], w[3]);
        }
    }
    publish<kStepDmas>();                               // the key near block has landed

    // ---- pass C: dq_rot = sum of weighted key rows (transposing reads of the permuted keys:
    // lane x gets element 4m + x, which is dim 16x + m) ----
    const int pt = 16 * wave + 4 * (pq >> 2) + x;
    const int kt = pq & 3;
    f4_t o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (f4_t){0.f, 0.f, 0.f, 0.f};
    {
        const int sv = pt - kt + kNear;
#pragma unroll
        for (int g = 0; g < kWG; ++g)
            if (4 * g <= W) row_sum_group(o, ww[g][0], ww[g][1], lds0, (sv - 4 * g) * kRowBytes, swz(sv - 4 * g));
        // near rung pairs: slot kt of the group is rung 2k + (kt >> 1), near row (kt even) at
        // pt + 64 - a, far row one slot down
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if constexpr (INT) {
                if ((k & 1) == 0 && k < kn) {
                    const int sl = pt + kNear - group_a(k, kt);
                    row_sum_group(o, wo[k][0], wo[k][1], lds0, sl * kRowBytes, swz(sl));
                }
            } else if (k < kn) {
                const int sl = pt + kNear - pick_uniform((kt >> 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a) - (kt & 1);
                row_sum_group(o, wo[k][0], wo[k][1], lds0, sl * kRowBytes, swz(sl));
            }
        }
        publish<0>();
    }
    {
        // (INT: the near rows of the step's rungs, slots pt and 72 + pt, each read twice)
        const int sv = INT ? pt + ((kt < 2) ? 0 : kBlkSlots) : (kt < 2) ? pt + 1 - kt : kBlkSlots + pt + 5 - kt;
        const int vbase = sv * kRowBytes, vsw = swz(sv);
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if (k >= kn && k < n_steps) {
                if (k + 1 < n_steps) step(krs, buf(k + 2), k + 1);
                row_sum_group(o, wo[k][0], wo[k][1], buf(k + 1), vbase, vsw);
                if (k + 1 < n_steps) publish<0>();
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- the key side's weights: the window row of this query (64 bytes; through treg as 16
    // rows per head, chunk c at c ^ x, 1 KB contiguous stores) and one entry of each rung's row
    // (rung-major, so a wave's stores of one rung are contiguous). dS is carried scaled by the
    // tile's 2^-ts (the largest row exponent of the head over the tile), known only after the
    // barrier below: a wave whose rows need no scaling (exponent 0) stores them ahead of it, and
    // stores them again, scaled, when another wave's rows set ts otherwise (the same lanes write
    // the same words, in order). (Pass C read only the key halves: treg is still the wave's own.)
    auto store_w = [&]() {
#pragma unroll
        for (int c = 0; c < kNW / 4; ++c)
            *reinterpret_cast<uint4*>(treg + (16 * x + pq) * (kNW * 4) + ((c ^ x) << 4)) =
                make_uint4(wq[4 * c], wq[4 * c + 1], wq[4 * c + 2], wq[4 * c + 3]);
        {
            // 4 LDS reads, then 4 buffer stores over the 4 heads' rows (a slot past L stores
            // beyond the buffer and is dropped, as in store_lin)
            const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
                A.wwin + (static_cast<int64_t>(b) * A.Hq + h0) * L * kNW, 0, 4 * L * kNW * 4, kRsrcWord3);
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sl = 16 * u + (lane >> 2), c = lane & 3;
                v[u] = *reinterpret_cast<const uint4*>(treg + sl * (kNW * 4) + ((c ^ u) << 4));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int sl = 16 * u + (lane >> 2), c = lane & 3;
                const int pos = i0 + 16 * wave + (sl & 15);
                const int off = pos < L ? ((sl >> 4) * L + pos) * (kNW * 4) + 16 * c : -(kNW * 4);
                typedef int v4i_t __attribute__((ext_vector_type(4)));
                const v4i_t d = {static_cast<int>(v[u].x), static_cast<int>(v[u].y), static_cast<int>(v[u].z), static_cast<int>(v[u].w)};
                __builtin_amdgcn_raw_buffer_store_b128(d, wrs, off, 0, 0);
            }
        }
        if (active) {
            uint32_t* rr = A.wrung + (static_cast<int64_t>(b) * A.Hq + h0 + x) * kNR * L + i;
            // rung n's entry: slot n (INT: n + ro past the near groups)
            auto wslot = [&](int y) -> uint32_t { return y < MAXK ? wq[4 * kWG + y] : 0u; };
#pragma unroll
            for (int n = 0; n < kNR; ++n) {
                uint32_t v = wslot(n);
                if constexpr (INT) {
                    // the candidates as register values first (a choice among the array's entries
                    // would become an indexed array in scratch memory)
                    uint32_t c1 = wslot(n + 1), c2 = wslot(n + 2), c3 = wslot(n + 3);
                    asm volatile("" : "+v"(v), "+v"(c1), "+v"(c2), "+v"(c3));
                    const int sh = n < nn ? 0 : ro;
                    v = sh == 0 ? v : sh == 1 ? c1 : sh == 2 ? c2 : c3;
                }
                rr[static_cast<int64_t>(n) * L] = v;
            }
        }
    };
    const bool wplain = !wave_any(es != kNoExp && es != 0);
    if (!or_votes(votes)) {
        if (wplain) store_w();
        {
            // ---- dq: to true units (head r's 2^ed from lane r of the quad), RoPE transposed at
            // position i. Lane x holds dims 16x + m of heads 0..3; the other half of pair
            // (16x + m) mod 32 is in lane x ^ 2. Rows go through treg: 1 KB contiguous stores ----
            // pair 16 (x & 1) + m: lane 2 (x & 1) + (m >> 3) holds it (each lane loads pairs
            // 8x..8x+7), at entry (m & 7) >> 1 of its quarter
            const float4* ct = reinterpret_cast<const float4*>(A.cstab) + static_cast<int64_t>(active ? i : 0) * (kPairs / 2) + 4 * x;
            float4 cq[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) cq[u] = ct[u];
            float2 cs[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float4& t = cq[(m & 7) >> 1];
                const float c = (m & 1) ? t.z : t.x, sn = (m & 1) ? t.w : t.y;
                cs[m] = (m < 8) ? make_float2(quad_f<kPerm0202>(c), quad_f<kPerm0202>(sn))
                                : make_float2(quad_f<kPerm1313>(c), quad_f<kPerm1313>(sn));
            }
            const float edf = pow2f(ed);
            const float eh[4] = {quad_f<kBcast0>(edf), quad_f<kBcast1>(edf), quad_f<kBcast2>(edf), quad_f<kBcast3>(edf)};
            const float sg = (x < 2) ? 1.f : -1.f;         // x' = x c + y s;  y' = y c - x s
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v[16];
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    const float other = quad_f<kXor2>(o[m][r]);
                    v[m] = fmaf(sg * other, cs[m].y, o[m][r] * cs[m].x);
                }
                if (wscaled) {
#pragma unroll
                    for (int m = 0; m < 16; ++m) v[m] *= eh[r];
                }
                uint4 lo, hi;
                lo.x = pack_bf2(v[0], v[1]);
                lo.y = pack_bf2(v[2], v[3]);
                lo.z = pack_bf2(v[4], v[5]);
                lo.w = pack_bf2(v[6], v[7]);
                hi.x = pack_bf2(v[8], v[9]);
                hi.y = pack_bf2(v[10], v[11]);
                hi.z = pack_bf2(v[12], v[13]);
                hi.w = pack_bf2(v[14], v[15]);
                *reinterpret_cast<uint4*>(treg + row_view_addr(pq, r, 2 * x)) = lo;
                *reinterpret_cast<uint4*>(treg + row_view_addr(pq, r, 2 * x + 1)) = hi;
            }
            store_lin(A.dq, treg, 2);
        }
    }

    // ---- d(loss)/dt partial sums of this workgroup (fixed order), and each head's largest dS
    // exponent over the tile ----
    if constexpr (PRECISE) {
#pragma unroll
        for (int n = 0; n < MAXK; ++n) {
            float v = active ? dt[n] : 0.f;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wave][n] = v;
        }
    }
    {
        const int ms = head_max(es);
        if (pq == 0) ered[wave][x][2] = ms;
    }
    // an LDS-only barrier: the stores in flight need not have landed (__syncthreads would wait
    // for every one of them)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int ts = max(max(ered[0][x][2], ered[1][x][2]), max(ered[2][x][2], ered[3][x][2]));
    if (ts == kNoExp) ts = 0;

    const int outside = or_votes(votes);
    if (threadIdx.x == 0) {
        if (blockIdx.x == 0) A.seqw[0] = A.seq;
        if (outside) A.seqw[1] = A.seq;
    }
    if (outside) {
        // the marker for the key side
        if (threadIdx.x < 4) A.exps[(static_cast<int64_t>(b) * A.Hq + h0 + x) * n_tiles + tile] = kExpsFallback;
    } else {
        if (!wplain || wave_any(es != kNoExp && es != ts)) {
            // dS from the row's exponent to the tile's
            const uint32_t fs = pow2_h2(0, es == kNoExp ? 0 : es - ts);
#pragma unroll
            for (int y = 0; y < 4 * kWG + MAXK; ++y) wq[y] = mul_h2(wq[y], fs);
            store_w();
        }
        if (PRECISE && threadIdx.x < static_cast<unsigned>(A.n_off)) {
            float v = 0.f;
            if (threadIdx.x < MAXK) v = ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x];
            A.partial[static_cast<int64_t>(blockIdx.x) * kMaxOff + threadIdx.x] = v;
        }
        // the tile's exponents of head x for the key side (and the call number, where they are not
        // all 0, for the key side to read them)
        if (threadIdx.x < 4) {
            const int tq = tile_exp(0), td = tile_exp(1);
            A.exps[(static_cast<int64_t>(b) * A.Hq + h0 + x) * n_tiles + tile] = pack_exps(tq, td, ts);
            if ((tq | td | ts) != 0) A.seqw[2] = A.seq;
        }
    }
}

// ------------------------------------------------------------------------------------------------
// The float32 tiles of the backward, after the matrix-core kernels. A query tile runs when the
// query kernel marked it (its exps words); a key tile runs when a query tile it reads from is
// marked (bwd_k_dot decides, and runs it in place of its own). The query tiles of a call run at
// the end of bwd_k_dot where the key stage runs in the same call, else in bwd_fp32_kernel; either
// way one load of the call numbers the query kernel leaves in the workspace skips them unless a
// tile of this call's query stage was marked. Workgroups stride over the query kernel's ones.
// ------------------------------------------------------------------------------------------------
// The marked query tiles of this call's query stage, workgroups first, first + stride, ... of the
// query kernel's n_qwg (its tile order: q_map is 0 or 1, which does not depend on the grid's size;
// virtual workgroup w takes the tile, and the partials slot, of that kernel's workgroup w).
__device__ __forceinline__ void query_fp32_tiles(const BwdArgs& A, int n_qwg, int q_map, int first, int stride, char* lds) {
    if (n_qwg <= 0 || !__builtin_amdgcn_readfirstlane(A.seqw[1] == A.seq ? 1 : 0)) return;
    const int n_tiles = (A.L + kTile - 1) / kTile;
    const int n_chunk = A.G >> 2;
    for (int w = first; w < n_qwg; w += stride) {
        int unit, tile;
        unit_tile(w, n_tiles, q_map, unit, tile);
        const int chunk = unit % n_chunk;
        const int bg = unit / n_chunk;
        const int b = bg / A.Hkv;
        const int h0 = (bg % A.Hkv) * A.G + chunk * 4;
        if (!(A.exps[(static_cast<int64_t>(b) * A.Hq + h0) * n_tiles + tile] & kExpsFallback)) continue;
        __syncthreads();                        // lds is free
        bwd_q_tile_fp32(A, b, bg, h0, tile * kTile, w, lds);
    }
}

constexpr int kFp32Grid = 1024;

// The query float32 tiles of a call whose key stage does not run.
__global__ __launch_bounds__(kNT) void bwd_fp32_kernel(BwdArgs A) {
    __shared__ __attribute__((aligned(16))) char lds[kTile * 16 * 4];
    query_fp32_tiles(A, A.q_fp32_wg, A.xcd_map, blockIdx.x, gridDim.x, lds);
}
// ------------------------------------------------------------------------------------------------
// bwd_k_dot. INT: every kept rung is integral (§2 "Implementation note"): a key row receives one
// query row per rung, so the rungs with a <= 64 come from the near block four to a group (at most
// two groups: terms te = 0..3 are four rungs' rows), and a far step stages 64-row blocks of its two
// rungs' rows, whose terms pair the two rungs at two elements per transposing read (one v_dot2 per
// element, half an interpolated step's).
// ------------------------------------------------------------------------------------------------
template <int MAXS, bool INT>
__global__ __launch_bounds__(kNT, 2) void bwd_k_dot_kernel(BwdArgs A) {
    // Two item buffers used in turn, each a rotated-query part and a do part (kBufBytes each).
    // Items of a query head: its near block (query rows j0 .. j0 + 127 of the rotated queries and
    // of do: the window and every rung pair with a <= 63), then its far steps (two larger rungs
    // each), padded to an odd count so that every head's near block sits in lds0. The near
    // block's buffer also holds the weights of the near rung pairs (2 KB after each part).
    __shared__ __attribute__((aligned(1024))) char lds0[2 * kBufBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[2 * kBufBytes];
    // a rung step's weights per key row: (dS near, dS far) of its two rungs, then (p near, p far)
    __shared__ uint4 wst[2][kTile];
    // the (p, dS) entries of a step's two rungs for queries j0 + a + 0..127 (step s: buffer s % 2),
    // staged by the item before the step's own
    __shared__ uint32_t went[2][2][128];
    // per head and query-tile slot: the factors (2^(td - Ev) low, 2^(ts + tq - Ek) high, fp16) that
    // bring the query side's per-tile scaling to the workgroup's common one (see below)
    constexpr int kSlotsF = 3 + 2 * 2 * MAXS;
    __shared__ uint32_t fac[kMaxGKey][kSlotsF];
    __shared__ int emax[4][2];                          // per wave: the common exponents Ev, Ek

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int L = A.L;
    const int n_tiles = (L + kTile - 1) / kTile;
    int unit, tile;
    unit_tile(blockIdx.x, n_tiles, A.xcd_map, unit, tile);
    const int bg = unit;                                // b * Hkv + g
    const int b = bg / A.Hkv, g = bg % A.Hkv;
    const int j0 = tile * kTile;

    // rungs some key row of the tile receives (query j + a < L): a prefix
    // (counted over the packed scan table, RungScan: a few wide scalar loads, where a loop over
    // the offset table waits for each rung's load in turn)
    int n_reach = 0, n_lo = 0;
#pragma unroll
    for (int n = 0; n < kScanRungs; ++n) {
        n_reach += (j0 + A.scan.a[n] < L) ? 1 : 0;
        n_lo += (A.scan.a[n] <= kNear - (INT ? 0 : 1)) ? 1 : 0;
    }
    // near rungs: the prefix with a <= 63 (both query rows of every key row of the tile inside the
    // near block; INT: a <= 64, the one row). Pairs k < kn come from the near block (kn even, at
    // most 4; INT: for even k a group of the four rungs 2k .. 2k + 3, those past nn padding);
    // pairs kn .. n_far - 1 are far steps, pair k in buffer (k + 1) % 2, n_far odd so that the last
    // one sits in lds1; far pair k holds rungs 2k - ro and 2k - ro + 1 (ro = 0 unless INT).
    const int n_near = min(n_lo, n_reach);
    const int nn = INT ? min(n_near, 8) : 0;
    const int kn = INT ? 2 * ((nn + 3) >> 2) : min((n_near >> 1) & ~1, 4);
    const int ro = INT ? 2 * kn - nn : 0;
    const int n_steps = INT ? kn + ((n_reach - nn + 1) >> 1) : (n_reach + 1) >> 1;
    const int n_far = max(n_steps, kn + 1) | 1;
    constexpr int kStepDmas = INT ? 4 : 6;              // DMA instructions per wave of a far step part

    // Lanes follow v_mfma_f32_16x16x16f16: lane l = 16 lg + lr holds A[lr][4 lg + 0..3],
    // B[4 lg + 0..3][lr] and D[4 lg + 0..3][lr]. Its outputs (window and rungs alike) are key rows
    // 16w + 4 lg + q (q = 0..3) at element E(nb, lr) of block nb = 0..3, where column t = 4b' + c
    // is element 8 ch + 4 (b' & 1) + c with chunk ch = nb + 4 (b' >> 1) (of the permuted rows of
    // the rotated queries for dk, of do for dv). With the slot swizzle, the transposing reads of
    // a pass of 32 lanes then fall on distinct banks.
    const int lr = lane & 15, lg = lane >> 4;
    const int tb = lr & 3, te = lr >> 2;                // as a source of a transposing read: block tb, row te
    f4_t dk[4], dv[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        dk[nb] = (f4_t){0.f, 0.f, 0.f, 0.f};
        dv[nb] = (f4_t){0.f, 0.f, 0.f, 0.f};
    }
    // byte offset of element block tb of block nb inside slot s
    auto blk_addr = [&](int s, int nb) { return (s * kRowBytes | (((nb + 4 * (tb >> 1)) << 4) ^ swz(s))) + 8 * (tb & 1); };

    Stager st;
    st.init(lane, wave);
    // rung step k: rung 2k rows j0 + a + s at slot s (near of key row r at r, far at r + 1), rung
    // 2k + 1 rows j0 + a' - 2 + s at slot 72 + s (near at 72 + r + 2, far at 72 + r + 3); steps past
    // n_steps stage zeros
    // (INT: 64 rows each, the row of key row r at slot r or 72 + r)
    auto step = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int k) {
        if constexpr (INT) {
            const int n = 2 * k - ro;
            st.step64(rs, dst, n < n_reach, j0 + A.off[n].a, n + 1 < n_reach, j0 + A.off[n + 1].a);
        } else {
            st.step(rs, dst, 2 * k < n_reach, j0 + A.off[2 * k].a, 2 * k + 1 < n_reach, j0 + A.off[2 * k + 1].a - 2);
        }
    };
    auto buf = [&](int it) -> char* { return (it & 1) ? lds1 : lds0; };
    // the rung entries of step k of head h into went[k % 2]: one 4-byte DMA per wave (rung
    // 2k + (w & 1), queries j0 + a + 64 (w >> 1) + lane; zeros past L or past the reach)
    auto entries = [&](int h, int k) {
        const int n = 2 * k - ro + (wave & 1);
        const bool real = n < n_reach;
        const uint32_t* wrn = A.wrung + ((static_cast<int64_t>(b) * A.Hq + h) * kNR + (real ? n : 0)) * L;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(wrn), 0, L * 4, kRsrcWord3);
        const int q0 = real ? j0 + A.off[n].a + 64 * (wave >> 1) : -(1 << 24);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dma_dst(reinterpret_cast<char*>(&went[k & 1][wave & 1][64 * (wave >> 1)])),
                                                 4, (q0 + lane) * 4, 0, 0, 0);
    };
    // the near item of head h: rotated-query and do rows j0 + s at slot s < 128 (4 + 4
    // instructions per wave) and the entries of far pair kn (1)
    auto near_item = [&](int h) {
        const int64_t hrow0 = (static_cast<int64_t>(b) * A.Hq + h) * L;
        st.near(rows_rsrc(A.qrot16, hrow0, L), lds0, j0);
        st.near(rows_rsrc(A.do16, hrow0, L), lds0 + kBufBytes, j0);
        entries(h, kn);
    };
    // the weights of near pair k (< 4) in lds0: 64 rows of 16 bytes after the near block's rows
    auto wnear = [&](int k) -> uint4* {
        return reinterpret_cast<uint4*>(lds0 + (k < 2 ? 0 : kBufBytes) + kNear * 2 * kRowBytes + (k & 1) * 1024);
    };
    // rung step weights: thread (row wrow, part wv) builds one word of wst for key row j0 + wrow:
    // rung 2k + (wv & 1), dS halves (wv < 2) or p halves, (near, far) times (1 - t, t)
    const int wrow = threadIdx.x >> 2, wv = threadIdx.x & 3;

    // 4 terms of key rows 16w + 4 lg + q at block nb: the lane reads (as a source) term te's row
    // at element block tb and receives the 4 terms' element E(nb, lr); two v_dot2 per element.
    // The reads are issued first; each result then passes an empty asm as a 64-bit value before it
    // is split into its two dwords (an optimisation has been seen to fold the second dword of the
    // read onto the first).
    const int rbase16 = 16 * wave + 4 * lg;
    // far steps: term te of key row r: near / far of rung 2k at slots r, r + 1, of rung 2k + 1 at
    // 74 + r, 75 + r; element block nb of it is at radr[q] ^ (nb << 4)
    // (INT: term te of key row r is rung 2k - ro + (te & 1), slot r or 72 + r, at element block
    // nb + (te >> 1) for the read of element blocks nb and nb + 1, nb even)
    int radr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        radr[q] = INT ? blk_addr(rbase16 + q + (te & 1) * kBlkSlots, 0) ^ ((te >> 1) << 4)
                      : blk_addr(rbase16 + q + (te & 1) + (te >> 1) * (kBlkSlots + 2), 0);
    // A step's sums run as passes of 8 transposing reads and their products, each pass's reads
    // issued before the previous pass's products, so that a wave multiplies with a pass of reads
    // in flight (the empty asm with a memory clobber keeps the reads ahead of the products).
    // Interpolated pass q0 (0 or 2): the terms of key rows q0 and q0 + 1 at element blocks 0..3.
    auto rung_reads = [&](unsigned long long (&rv)[8], const char* lds, const int (&adr)[4], int q0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + (u >> 2), nb = u & 3;
            rv[u] = __builtin_bit_cast(unsigned long long, tr_read_h4(lds, adr[q] ^ (nb << 4)));
        }
    };
    auto rung_products = [&](f4_t (&acc)[4], const uint4 (&w)[4], bool use_p, unsigned long long (&rv)[8], int q0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = q0 + (u >> 2), nb = u & 3;
            asm volatile("" : "+v"(rv[u]));
            const uint32_t lo = static_cast<uint32_t>(rv[u]), hi = static_cast<uint32_t>(rv[u] >> 32);
            const uint32_t w01 = use_p ? w[q].z : w[q].x, w23 = use_p ? w[q].w : w[q].y;
            acc[nb][q] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w01), __builtin_bit_cast(h2_t, lo), acc[nb][q], false);
            acc[nb][q] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w23), __builtin_bit_cast(h2_t, hi), acc[nb][q], false);
        }
    };
    auto ahead = [] { asm volatile("" ::: "memory"); };
    // dk and dv rung sums of one step: its rotated-query part at lds, its do part kBufBytes on
    auto sum_rungs = [&](const uint4 (&w)[4], const char* lds, const int (&adr)[4]) {
        unsigned long long ra[8], rb[8];
        rung_reads(ra, lds, adr, 0);
        rung_reads(rb, lds, adr, 2);
        ahead();
        rung_products(dk, w, false, ra, 0);
        rung_reads(ra, lds + kBufBytes, adr, 0);
        ahead();
        rung_products(dk, w, false, rb, 2);
        rung_reads(rb, lds + kBufBytes, adr, 2);
        ahead();
        rung_products(dv, w, true, ra, 0);
        rung_products(dv, w, true, rb, 2);
    };

    // INT far steps: one read gives the two rungs' elements E(nb) and E(nb + 1) (nb even); the
    // weight word pairs the two rungs (dS halves in w.x, p halves in w.z)
    auto pair_reads = [&](unsigned long long (&rv)[8], const char* lds, const int (&adr)[4]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = u >> 1, nb = 2 * (u & 1);
            rv[u] = __builtin_bit_cast(unsigned long long, tr_read_h4(lds, adr[q] ^ (nb << 4)));
        }
    };
    auto pair_products = [&](f4_t (&acc)[4], const uint4 (&w)[4], bool use_p, unsigned long long (&rv)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int q = u >> 1, nb = 2 * (u & 1);
            asm volatile("" : "+v"(rv[u]));
            const uint32_t lo = static_cast<uint32_t>(rv[u]), hi = static_cast<uint32_t>(rv[u] >> 32);
            const h2_t wab = __builtin_bit_cast(h2_t, use_p ? w[q].z : w[q].x);
            acc[nb][q] = __builtin_amdgcn_fdot2(wab, __builtin_bit_cast(h2_t, lo), acc[nb][q], false);
            acc[nb + 1][q] = __builtin_amdgcn_fdot2(wab, __builtin_bit_cast(h2_t, hi), acc[nb + 1][q], false);
        }
    };
    auto sum_pairs = [&](const uint4 (&w)[4], const char* lds, const int (&adr)[4]) {
        unsigned long long ra[8], rb[8];
        pair_reads(ra, lds, adr);
        pair_reads(rb, lds + kBufBytes, adr);
        ahead();
        pair_products(dk, w, false, ra);
        pair_products(dv, w, true, rb);
    };

    // ---- the query side scaled each head's rows of a query tile by powers of two of the tile's
    // own (q by 2^-tq, do by 2^-td, dS by 2^-ts; exps). Per head, slot s < 3 is query tile t0 + s
    // (the window and the near pairs), slot 3 + 2n + u is tile ((j0 + a_n) >> 6) + u (rung n). Ev
    // and Ek are the largest td and ts + tq over the workgroup's heads and slots, and each weight
    // takes its query tile's factor 2^(td - Ev) (p) or 2^(ts + tq - Ek) (dS), at most 1: dv and dk
    // accumulate in units of 2^-Ev and 2^-Ek, scaled back at the end. The query stage leaves its
    // call number in seqw[1] when a tile fell back to float32 and in seqw[2] when some tile's
    // exponents are not all 0; where neither holds (the usual case: rows fp16 holds as they are
    // carry exponent 0) every factor is 1 and no exponent is read. Every wave builds the whole
    // table (the same words), so no barrier is needed; the weights always take their factors
    // (multiplies without branches). ----
    const int t0 = tile;
    const uint64_t seq_last = A.seqw[0], seq_fb = A.seqw[1], seq_sc = A.seqw[2];
    near_item(g * A.G);
    bool allone = true;                                 // uniform: every factor of the table is 1
    // the table; false when a query tile this tile reads from left its hand-off to the float32
    // tiles (then so does this one)
    auto build_factors = [&]() -> bool {
        constexpr int kFacLoads = (kMaxGKey * kSlotsF + 63) / 64;
        if (__builtin_amdgcn_readfirstlane((seq_fb != seq_last && seq_sc != seq_last) ? 1 : 0)) {
#pragma unroll
            for (int r = 0; r < kFacLoads; ++r) {
                const int e = lane + 64 * r;
                if (e < kMaxGKey * kSlotsF) fac[e / kSlotsF][e % kSlotsF] = 0x3c003c00u;   // (1, 1)
            }
            if (lane == 0) emax[wave][0] = emax[wave][1] = 0;
            return true;
        }
        uint32_t ew[kFacLoads];
#pragma unroll
        for (int r = 0; r < kFacLoads; ++r) {
            const int e = lane + 64 * r;
            const int hh = e / kSlotsF, sl = e % kSlotsF;
            int tl = t0 + sl;
            bool ok = hh < A.G;
            if (sl >= 3) {
                const int n = (sl - 3) >> 1;
                int a = 0;
#pragma unroll
                for (int m = 0; m < 2 * MAXS; ++m) a = (n == m) ? A.off[m].a : a;   // uniform table, lane's pick
                tl = ((j0 + a) >> 6) + ((sl - 3) & 1);
                ok = ok && n < n_reach;
            }
            ok = ok && tl < n_tiles;
            ew[r] = ok ? A.exps[(static_cast<int64_t>(b) * A.Hq + g * A.G + hh) * n_tiles + tl] : 0xffffffffu;
        }
        int mv = kNoExp, mk = kNoExp;
        bool marked = false;
#pragma unroll
        for (int r = 0; r < kFacLoads; ++r) {
            if (ew[r] != 0xffffffffu) {
                mv = max(mv, exps_td(ew[r]));
                mk = max(mk, exps_ts(ew[r]) + exps_tq(ew[r]));
                marked = marked || (ew[r] & kExpsFallback) != 0u;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            mv = max(mv, __shfl_xor(mv, off, 64));
            mk = max(mk, __shfl_xor(mk, off, 64));
        }
        if (wave_any(marked)) return false;
        const int Ev = __builtin_amdgcn_readfirstlane(mv == kNoExp ? 0 : mv);
        const int Ek = __builtin_amdgcn_readfirstlane(mk == kNoExp ? 0 : mk);
        if (lane == 0) {
            emax[wave][0] = Ev;
            emax[wave][1] = Ek;
        }
        bool other = false;
#pragma unroll
        for (int r = 0; r < kFacLoads; ++r) {
            const int e = lane + 64 * r;
            const bool real = ew[r] != 0xffffffffu;
            other = other || (real && (exps_td(ew[r]) != Ev || exps_ts(ew[r]) + exps_tq(ew[r]) != Ek));
            if (e < kMaxGKey * kSlotsF)
                fac[e / kSlotsF][e % kSlotsF] = real ? pow2_h2(exps_td(ew[r]) - Ev, exps_ts(ew[r]) + exps_tq(ew[r]) - Ek) : 0u;
        }
        allone = !wave_any(other);
        return true;
    };
    // the factor of one entry half: p (use_p) or dS, of head hh's slot sl, as an fp16 in the low 16 bits
    auto fac_half = [&](int hh, int sl, bool use_p) -> uint32_t {
        const uint32_t f = fac[hh][sl];
        return use_p ? (f & 0xffffu) : (f >> 16);
    };
    // (1 - t, t) times the factors of the near and far query rows of rung n for key row j0 + wrow
    auto coef = [&](int hh, int n, int a, float t, bool use_p) -> h2_t {
        const h2_t c = {static_cast<_Float16>(1.f - t), static_cast<_Float16>(t)};
        const int qn = j0 + wrow + a;
        const int base = (n < 2 * kn) ? -t0 : 3 + 2 * n - ((j0 + a) >> 6);
        const uint32_t f = fac_half(hh, base + (qn >> 6), use_p) | (fac_half(hh, base + ((qn + 1) >> 6), use_p) << 16);
        return c * __builtin_bit_cast(h2_t, f);
    };
    // the thread's coefficient of each rung pair k (rung 2k + (wv & 1), dS halves for wv < 2, else
    // p halves): (1 - t, t), times the factors of its near and far query rows where not every
    // factor is 1 (then recomputed per head)
    // INT: no (1 - t, t): a word pairs two rungs, each with its own query row's factor; a near
    // group (even k < kn) rungs 2k + 2 (wv & 1) and the next, a far pair k rungs 2k - ro and the next
    auto near_a = [&](int k, int c) -> int { return 2 * k + c < nn ? A.off[2 * k + c].a : 0; };
    uint32_t cw[MAXS];
    auto set_cw = [&](int hh, bool with_factors) {
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if constexpr (INT) {
                const bool use_p = (wv >> 1) != 0;
                if (k < kn) {
                    const int a0 = pick_uniform((wv & 1) != 0, near_a(k, 2), near_a(k, 0));
                    const int a1 = pick_uniform((wv & 1) != 0, near_a(k, 3), near_a(k, 1));
                    const uint32_t f = with_factors ? fac_half(hh, ((j0 + wrow + a0) >> 6) - t0, use_p) |
                                                          (fac_half(hh, ((j0 + wrow + a1) >> 6) - t0, use_p) << 16)
                                                    : 0x3c003c00u;
                    cw[k] = f;
                } else {
                    const int n = 2 * k - ro;
                    const int a0 = A.off[n].a, a1 = A.off[n + 1].a;
                    cw[k] = with_factors ? fac_half(hh, 3 + 2 * n + ((j0 + wrow + a0) >> 6) - ((j0 + a0) >> 6), use_p) |
                                               (fac_half(hh, 5 + 2 * n + ((j0 + wrow + a1) >> 6) - ((j0 + a1) >> 6), use_p) << 16)
                                         : 0x3c003c00u;
                }
            } else {
                const float t = pick_uniform((wv & 1) != 0, A.off[2 * k + 1].t, A.off[2 * k].t);
                const int a = pick_uniform((wv & 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a);
                const h2_t c = with_factors ? coef(hh, 2 * k + (wv & 1), a, t, (wv >> 1) != 0)
                                            : (h2_t){static_cast<_Float16>(1.f - t), static_cast<_Float16>(t)};
                cw[k] = __builtin_bit_cast(uint32_t, c);
            }
        }
    };
    set_cw(0, false);
    // rung step weights of head hh: thread (row wrow, part wv) builds one word of wst for key row
    // j0 + wrow: rung 2k + (wv & 1), dS halves (wv < 2) or p halves, times the coefficient
    // (INT: the entries of the pair's two rungs at their near query rows, for every wv)
    auto put_w = [&](int k) {
        const uint32_t en = went[k & 1][INT ? 0 : wv & 1][wrow], ef = went[k & 1][INT ? 1 : wv & 1][wrow + (INT ? 0 : 1)];
        const uint32_t pr = __builtin_amdgcn_perm(ef, en, (wv >> 1) ? 0x05040100u : 0x07060302u);
        reinterpret_cast<uint32_t*>(&wst[k & 1][wrow])[wv] = mul_h2(pr, cw[k]);
    };

    if (!__builtin_amdgcn_readfirstlane(build_factors() ? 1 : 0)) {
        // a query tile this tile reads from left its hand-off to the float32 tiles: so does this
        // one (the staging in flight lands first)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        bwd_k_tile_fp32(A, b, bg, g, j0);
        query_fp32_tiles(A, A.q_fp32_wg, A.q_xcd_map, blockIdx.x, gridDim.x, lds0);
        return;
    }
    for (int hh = 0; hh < A.G; ++hh) {
        const int h = g * A.G + hh;
        const int64_t hrow0 = (static_cast<int64_t>(b) * A.Hq + h) * L;
        const __amdgpu_buffer_rsrc_t qrs = rows_rsrc(A.qrot16, hrow0, L);
        const __amdgpu_buffer_rsrc_t drs = rows_rsrc(A.do16, hrow0, L);
        // window weights of the wave's key rows 16w + lr and queries 16w + c (c = 16 kb + 4 lg +
        // ee), distance c - lr (zero outside 0..15 or past L), and the (p, dS) entries of the near
        // pairs for the weight table below: loaded before this head's first DMA (loads count in
        // vmcnt with the DMAs, in issue order)
        uint32_t e4w[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ee = 0; ee < 4; ++ee) {
                const int c = 16 * kb + 4 * lg + ee;
                const int d = c - lr;
                const int qr = j0 + 16 * wave + c;
                const bool ok = d >= 0 && d < kNW && qr < L;
                const uint32_t v = A.wwin[(hrow0 + (ok ? qr : 0)) * kNW + (d & 15)];
                e4w[kb][ee] = ok ? v : 0u;
            }
        }
        uint32_t enr[4], efr[4];
        {
            const uint32_t* wr = A.wrung + hrow0 * kNR;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if constexpr (INT) {
                    // group k (even): rungs n0 = 2k + 2 (wv & 1) and n0 + 1 at their query rows
                    const int n0 = 2 * k + 2 * (wv & 1);
                    const int q0 = j0 + wrow + pick_uniform((wv & 1) != 0, near_a(k, 2), near_a(k, 0));
                    const int q1 = j0 + wrow + pick_uniform((wv & 1) != 0, near_a(k, 3), near_a(k, 1));
                    const bool ok0 = (k & 1) == 0 && k < kn && n0 < nn && q0 < L;
                    const bool ok1 = (k & 1) == 0 && k < kn && n0 + 1 < nn && q1 < L;
                    const uint32_t v0 = wr[static_cast<int64_t>(ok0 ? n0 : 0) * L + (ok0 ? q0 : 0)];
                    const uint32_t v1 = wr[static_cast<int64_t>(ok1 ? n0 + 1 : 0) * L + (ok1 ? q1 : 0)];
                    enr[k] = ok0 ? v0 : 0u;
                    efr[k] = ok1 ? v1 : 0u;
                } else {
                    const int n = 2 * k + (wv & 1);
                    const int qn = j0 + wrow + pick_uniform((wv & 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a);
                    const bool okn = k < kn && qn < L, okf = k < kn && qn + 1 < L;
                    const uint32_t vn = wr[static_cast<int64_t>(n) * L + (okn ? qn : 0)];
                    const uint32_t vf = wr[static_cast<int64_t>(n) * L + (okf ? qn + 1 : 0)];
                    enr[k] = okn ? vn : 0u;
                    efr[k] = okf ? vf : 0u;
                }
            }
        }
        step(qrs, lds1, kn);
        step(drs, lds1 + kBufBytes, kn);
        entries(h, kn + 1);
        if (!__builtin_amdgcn_readfirstlane(allone ? 1 : 0)) set_cw(hh, true);
        // the near pairs' weights (same words as the far steps' table; INT: the groups', even k)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < kn && (!INT || (k & 1) == 0)) {
                const uint32_t pr = __builtin_amdgcn_perm(efr[k], enr[k], (wv >> 1) ? 0x05040100u : 0x07060302u);
                reinterpret_cast<uint32_t*>(&wnear(k)[wrow])[wv] = mul_h2(pr, cw[k]);
            }
        }
        // the window's factors: the wave's queries 16w + 16 kb + 0..15 lie in query tile t0, but
        // for wave 3, kb = 1 (tile t0 + 1)
        const uint32_t fw0 = fac[hh][0], fw1 = fac[hh][wave == 3 ? 1 : 0];
        publish<2 * kStepDmas + 1>();                   // this head's near item and weights are in place

        // ---- window terms on the matrix cores: for the wave's key rows 16w + rr and queries
        // 16w + c (c < 32), dk_rot[rr] += sum_c A[rr][c] qrot[c], A[rr][c] = dS of query c at
        // distance c - rr (zero outside 0..15); dv likewise with p and do ----
        {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                // each query's (p, dS) pair times its query tile's factors
                uint32_t e4[4];
#pragma unroll
                for (int ee = 0; ee < 4; ++ee) e4[ee] = mul_h2(e4w[kb][ee], kb ? fw1 : fw0);
                // (p, dS) pairs: dS in the high halves (dk), p in the low halves (dv)
                const u2_t a_dk = {__builtin_amdgcn_perm(e4[1], e4[0], 0x07060302u),
                                   __builtin_amdgcn_perm(e4[3], e4[2], 0x07060302u)};
                const u2_t a_dv = {__builtin_amdgcn_perm(e4[1], e4[0], 0x05040100u),
                                   __builtin_amdgcn_perm(e4[3], e4[2], 0x05040100u)};
                const int slot = 16 * wave + 16 * kb + 4 * lg + te;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const h4_t bq = tr_read_h4(lds0, blk_addr(slot, nb));
                    const h4_t bd = tr_read_h4(lds0 + kBufBytes, blk_addr(slot, nb));
                    dk[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a_dk), bq, dk[nb], 0, 0, 0);
                    dv[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a_dv), bd, dv[nb], 0, 0, 0);
                }
            }
        }
        // ---- near rung pairs: term te of key row r is rung 2k + (te >> 1), near row j + a at
        // slot r + a (te even) or far row one slot up ----
        // (INT, even k: term te is rung 2k + te, query row j + a at slot r + a)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (k < kn && (!INT || (k & 1) == 0)) {
                int nadr[4];
                if constexpr (INT) {
                    const int ak = pick4(te, near_a(k, 0), near_a(k, 1), near_a(k, 2), near_a(k, 3));
#pragma unroll
                    for (int q = 0; q < 4; ++q) nadr[q] = blk_addr(rbase16 + q + ak, 0);
                } else {
                    const int ak = pick_uniform((te >> 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a);
#pragma unroll
                    for (int q = 0; q < 4; ++q) nadr[q] = blk_addr(rbase16 + q + ak + (te & 1), 0);
                }
                uint4 w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = wnear(k)[rbase16 + q];
                sum_rungs(w, lds0, nadr);
            }
        }
        put_w(kn);
        publish<0>();                                   // far pair kn and its weights are in place, lds0 is free

        // ---- far steps: pair k (kn <= k < n_far) in lds(k + 1) % 2 ----
#pragma unroll
        for (int k = 0; k < MAXS + 1; ++k) {
            if (k >= kn && k < n_far) {
                if (k + 1 < n_far) {
                    step(qrs, buf(k + 2), k + 1);
                    step(drs, buf(k + 2) + kBufBytes, k + 1);
                    entries(h, k + 2);
                } else if (hh + 1 < A.G) {
                    near_item(h + 1);                   // the last item sits in lds1
                }
                if (k < n_steps) {
                    uint4 w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[q] = wst[k & 1][rbase16 + q];
                    if constexpr (INT) {
                        sum_pairs(w, buf(k + 1), radr);
                    } else {
                        sum_rungs(w, buf(k + 1), radr);
                    }
                }
                if (k + 1 < n_steps) put_w(k + 1);
                publish<0>();
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // to true units (the weights carried 2^-Ek and 2^-Ev)
    {
        const float fk = pow2f(emax[wave][1]), fv = pow2f(emax[wave][0]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            dk[nb] *= fk;
            dv[nb] *= fv;
        }
    }

    // ---- dk: RoPE transposed at each key position. Element 4m + c of the permuted rows is dim
    // 16c + m; the lane's element E = 8 ch + 4 (b' & 1) + c is dim 16c + 2 ch + (b' & 1); its
    // pair partner (dim +- 32) is element E ^ 2, in lane lr ^ 2 ----
    {
        const int bq_ = lr >> 2, c = lr & 3;
        const float sg = (c < 2) ? 1.f : -1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int jr = j0 + rbase16 + q;
            const float2* cs = reinterpret_cast<const float2*>(A.cstab) + static_cast<int64_t>(jr < L ? jr : 0) * kPairs;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int ch = nb + 4 * (bq_ >> 1);
                const int pair = (16 * c + 2 * ch + (bq_ & 1)) & 31;
                const float2 t = cs[pair];
                const float other = quad_f<kXor2>(dk[nb][q]);
                dk[nb][q] = fmaf(sg * other, t.y, dk[nb][q] * t.x);
            }
        }
    }
    // ---- regroup through LDS into rows of 64 dims (bf16), then 16-byte stores ----
    {
        bf16_t* tk = reinterpret_cast<bf16_t*>(lds0);
        bf16_t* tv = reinterpret_cast<bf16_t*>(lds1);
        const int bq_ = lr >> 2, c = lr & 3;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            const int ch = nb + 4 * (bq_ >> 1);
            const int ek = 16 * c + 2 * ch + (bq_ & 1);                 // dim of the element (dk and dv)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = rbase16 + q;
                tk[row * kD + ek] = static_cast<bf16_t>(pack_bf2(dk[nb][q], 0.f) & 0xffffu);
                tv[row * kD + ek] = static_cast<bf16_t>(pack_bf2(dv[nb][q], 0.f) & 0xffffu);
            }
        }
    }
    __syncthreads();
    {
        const int row = threadIdx.x >> 2, part = threadIdx.x & 3;      // 16 dims of one row
        const int j = j0 + row;
        if (j < L) {
            const int64_t orow = (static_cast<int64_t>(bg) * L + j) * kD + 16 * part;
            const uint4* sk = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(lds0) + row * kD + 16 * part);
            const uint4* sv = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(lds1) + row * kD + 16 * part);
            bf16_t* gk = static_cast<bf16_t*>(A.dk) + orow;
            bf16_t* gv = static_cast<bf16_t*>(A.dv) + orow;
            store_nt(gk, sk[0]);
            store_nt(gk + 8, sk[1]);
            store_nt(gv, sv[0]);
            store_nt(gv + 8, sv[1]);
        }
    }
    // the query tiles this call's query stage left to float32
    query_fp32_tiles(A, A.q_fp32_wg, A.q_xcd_map, blockIdx.x, gridDim.x, lds0);
}

}  // namespace

bool bwd_mfma_supported(const BwdArgs& A) {
    return A.G % 4 == 0 && A.G <= kMaxGKey && A.W <= 15 && A.n_off <= 16;
}

hipError_t launch_bwd_mfma(const BwdArgs& A0, bool want_dalpha, int stages, hipStream_t s) {
    static std::atomic<uint64_t> calls{0};
    BwdArgs A = A0;
    A.seq = calls.fetch_add(1, std::memory_order_relaxed) + 1;
    const int64_t n_tiles = (A.L + kTile - 1) / kTile;
    const int64_t q_units = static_cast<int64_t>(A.B) * A.Hkv * (A.G / 4);
    const int64_t k_units = static_cast<int64_t>(A.B) * A.Hkv;
    A.n_wg = static_cast<int32_t>(q_units * n_tiles);
    const int q_map = (q_units % 8 == 0) ? 1 : 0;
    hipError_t e;
    if (stages & kStageQuery) {
        A.xcd_map = q_map;
        const dim3 grid(static_cast<unsigned>(q_units * n_tiles));
        if (want_dalpha)
            hipLaunchKernelGGL((bwd_q_mfma_kernel<8, true, false>), grid, dim3(kNT), 0, s, A);
        else if (int_path_fits(A.off, A.n_off, 8))
            hipLaunchKernelGGL((bwd_q_mfma_kernel<8, false, true>), grid, dim3(kNT), 0, s, A);
        else
            hipLaunchKernelGGL((bwd_q_mfma_kernel<8, false, false>), grid, dim3(kNT), 0, s, A);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the query float32 tiles run at the end of the key kernel where it runs in this call
    A.q_fp32_wg = (stages & kStageQuery) ? static_cast<int32_t>(q_units * n_tiles) : 0;
    A.q_xcd_map = q_map;
    if (stages & kStageKey) {
        A.xcd_map = (k_units % 32 == 0) ? 3 : (k_units % 8 == 0) ? 1 : 0;   // 3: heavy (low) key tiles first
        if (int_path_fits(A.off, A.n_off, 8))
            hipLaunchKernelGGL((bwd_k_dot_kernel<8, true>), dim3(static_cast<unsigned>(k_units * n_tiles)), dim3(kNT), 0, s,
                               A);
        else
            hipLaunchKernelGGL((bwd_k_dot_kernel<8, false>), dim3(static_cast<unsigned>(k_units * n_tiles)), dim3(kNT), 0, s,
                           A);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((stages & kStageQuery) && !(stages & kStageKey)) {
        A.xcd_map = q_map;
        const int64_t grid = std::min<int64_t>(q_units * n_tiles, kFp32Grid);
        hipLaunchKernelGGL(bwd_fp32_kernel, dim3(static_cast<unsigned>(grid)), dim3(kNT), 0, s, A);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((stages & kStageKey) && want_dalpha) return launch_dalpha(A, s);
    return hipSuccess;
}

}  // namespace fibattn
