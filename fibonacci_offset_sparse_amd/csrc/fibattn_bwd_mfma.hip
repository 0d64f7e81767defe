// Backward pass for bfloat16 storage on gfx950: the query side on the matrix cores, the key side
// with packed dot products, both streaming shifted row blocks through LDS.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv
// 2606.28560): §2 "Attended set" (window distances 0..W plus one slot per rung at d = alpha f,
// read by linear interpolation between rows i - floor(d) and i - floor(d) - 1, RoPE before the
// gather) and §2 "Per-layer scalar" (alpha = 0.5 + sigmoid(theta): the interpolation weight t is
// what carries a gradient to alpha). Gradients are of sum(do * o).
//
// Inputs come from prep_kv16's backward layout: rotated keys with dims permuted (element 4m + c of
// a row holds dim 16c + m) and values in dim order, fp16, plus the cos/sin table.
//
//  * bwd_q_mfma: workgroup = (batch, kv head, 4 query heads, 64 positions), lanes as in the forward
//    (fibattn_mfma.h). Three passes over the staged blocks:
//      A, keys: scores s (base 2), recomputed in fp32 from fp16 operands, and for every rung the
//         difference far - near of the two row products;
//      B, values: dP = do . value row, and far - near of it; then in registers p = softmax(s),
//         delta = sum p dP, dS = p (dP - delta), and the d(loss)/dt terms
//         dS (q . (k_far - k_near)) / sqrt(D) + p do . (v_far - v_near);
//      C, keys: dq_rot = sum dS/sqrt(D) (coefficient) key row, with transposing reads of the
//         permuted keys (a lane then holds 16 consecutive dims of 4 heads), RoPE transposed
//         between lanes x and x ^ 2, written as dq.
//    It also writes the rotated queries (fp16, permuted), do as fp16 and, per key row and term,
//    the weights the key side needs: p times the term's coefficient and dS/sqrt(D) times it, both
//    fp16.
//  * bwd_k_dot: workgroup = (batch, kv head, 64 key rows). Key row j is read by query j + delta of
//    every term (window distance d; the near row of a rung at a, coefficient 1 - t; its far row at
//    a + 1, coefficient t): for each query head, shifted blocks of rotated queries and of do are
//    staged and dk_rot[j] += w_ds q_rot, dv[j] += w_p do accumulate 4 terms at a time from
//    transposing reads (a lane gets 4 rows' element 4m + x) with two v_dot2 per element.
//  * dalpha (fibattn_bwd.hip): fixed-order sum of the per-workgroup dt partials.
// No atomics: results are bitwise reproducible.
#include "fibattn_mfma.h"

namespace fibattn {

namespace {

using namespace mx;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;

// fp16 p in the low half, fp16 ds in the high half (bf16 p loses too much of dv: 2^-9 per term)
__device__ __forceinline__ uint32_t pack_p_ds(float p, float ds) { return pack_h2(p, ds); }

// ------------------------------------------------------------------------------------------------
// bwd_q_mfma
// ------------------------------------------------------------------------------------------------
template <int MAXS>
__global__ __launch_bounds__(kNT, 2) void bwd_q_mfma_kernel(BwdArgs A) {
    constexpr int MAXK = 2 * MAXS;
    __shared__ __attribute__((aligned(1024))) char lds0[kBufBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[kBufBytes];
    __shared__ float red[4][MAXK];

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

    int n_reach = 0;
    for (int n = 0; n < A.n_off; ++n)
        if (i0 + kTile - 1 >= A.off[n].a + A.off[n].interp) n_reach = n + 1;
    const int n_steps = (n_reach + 1) >> 1;

    const int64_t kv_row0 = static_cast<int64_t>(bg) * L;
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(A.kstage, kv_row0, L);
    const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(A.vstage, kv_row0, L);
    Stager st;
    st.init(lane, wave);
    auto step = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int k) {
        st.step(rs, dst, 2 * k < n_reach, i0 - A.off[2 * k].a - 1, 2 * k + 1 < n_reach, i0 - A.off[2 * k + 1].a - 3);
    };
    auto buf = [&](int j) -> char* { return (j & 1) ? lds1 : lds0; };
    const int jw = i0 - W - kWinPad;

    // ---- prologue: key window, q and do of head h0 + x, key step 0 ----
    st.window(krs, lds0, jw);
    const int64_t qrow = (static_cast<int64_t>(b) * A.Hq + h0 + x) * L + (active ? i : 0);
    uint4 qraw[8], draw[8];
    float4 ctab[16];
    {
        const bf16_t* qr = static_cast<const bf16_t*>(A.q) + qrow * kD;
        const bf16_t* dr = static_cast<const bf16_t*>(A.dout) + qrow * kD;
#pragma unroll
        for (int c = 0; c < 8; ++c) qraw[c] = *reinterpret_cast<const uint4*>(qr + 8 * c);
#pragma unroll
        for (int c = 0; c < 8; ++c) draw[c] = *reinterpret_cast<const uint4*>(dr + 8 * c);
        const float4* ct = reinterpret_cast<const float4*>(A.cstab) + static_cast<int64_t>(active ? i : 0) * (kPairs / 2);
#pragma unroll
        for (int u = 0; u < 16; ++u) ctab[u] = ct[u];
    }
    step(krs, lds1, 0);

    // q rotated at its position (unscaled), fp16, in the keys' permuted order: word 2m holds dims
    // (m, 16 + m), word 2m + 1 dims (32 + m, 48 + m); register chunk c = words 4c..4c+3
    uint32_t q[8][4];
    {
        float r[kD];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t lw[4] = {qraw[c].x, qraw[c].y, qraw[c].z, qraw[c].w};
            const uint32_t hw[4] = {qraw[c + 4].x, qraw[c + 4].y, qraw[c + 4].z, qraw[c + 4].w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 t = ctab[4 * c + m];      // pairs 8c + 2m, 8c + 2m + 1
                const float x0 = bf16_lo(lw[m]), x1 = bf16_hi(lw[m]);
                const float y0 = bf16_lo(hw[m]), y1 = bf16_hi(hw[m]);
                const int j = 8 * c + 2 * m;
                r[j] = x0 * t.x - y0 * t.y;
                r[j + 1] = x1 * t.z - y1 * t.w;
                r[j + 32] = y0 * t.x + x0 * t.y;
                r[j + 33] = y1 * t.z + x1 * t.w;
            }
        }
#pragma unroll
        for (int w = 0; w < 32; ++w) {
            const int m = w >> 1;
            q[w >> 2][w & 3] = (w & 1) ? pack_h2(r[32 + m], r[48 + m]) : pack_h2(r[m], r[16 + m]);
        }
    }
    // do as fp16 in dim order (the values are staged in dim order)
    uint32_t dov[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t w4[4] = {draw[c].x, draw[c].y, draw[c].z, draw[c].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) dov[c][u] = pack_h2(bf16_lo(w4[u]), bf16_hi(w4[u]));
    }
    publish<6>();                                       // the key window has landed

    // ---- pass A: scores (base 2) and far - near of the rung products ----
    float s[4 * kWG + MAXK], sd[MAXK];
    const int s0 = p - x + W + kWinPad;                 // window: lane x reads distance 4g + x
    const int rslot = p + ((x >> 1) ? kBlkSlots + 2 : 0) + ((x & 1) ? 0 : 1);   // rung rows
    const int rbase = rslot * kRowBytes, rsw = swz(rslot);
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
        f4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (4 * g <= W) acc = row_dot_group(q, lds0, (s0 - 4 * g) * kRowBytes, swz(s0 - 4 * g));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = 4 * g + r;
            s[d] = (active && d <= W && i >= d) ? acc[r] * A.qscale : kNegInf;
        }
    }
    // (stores count in vmcnt too: issued where the next wait drains everything anyway)
    if (active) {
        uint4* qo = reinterpret_cast<uint4*>(static_cast<f16_t*>(A.qrot16) + qrow * kD);
#pragma unroll
        for (int c = 0; c < 8; ++c) qo[c] = make_uint4(q[c][0], q[c][1], q[c][2], q[c][3]);
        uint4* dq16 = reinterpret_cast<uint4*>(static_cast<f16_t*>(A.do16) + qrow * kD);
#pragma unroll
        for (int c = 0; c < 8; ++c) dq16[c] = make_uint4(dov[c][0], dov[c][1], dov[c][2], dov[c][3]);
    }
    publish<0>();
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            s[4 * kWG + 2 * k + e] = kNegInf;
            sd[2 * k + e] = 0.f;
        }
        if (k < n_steps) {
            if (k + 1 < n_steps) step(krs, buf(k + 2), k + 1);
            const f4_t acc = row_dot_group(q, buf(k + 1), rbase, rsw);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int n = 2 * k + e;
                if (n < n_reach) {
                    const float dd = (acc[2 * e + 1] - acc[2 * e]) * A.qscale;
                    const float sc = fmaf(A.off[n].t, dd, acc[2 * e] * A.qscale);
                    const bool ok = active && i >= A.off[n].a + A.off[n].interp;
                    s[4 * kWG + n] = ok ? sc : kNegInf;
                    sd[n] = ok ? dd : 0.f;
                }
            }
            publish<0>();
        }
    }

    // ---- value window and value step 0 under the softmax ----
    st.window(vrs, lds0, jw);
    step(vrs, lds1, 0);
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
    publish<6>();

    // ---- pass B: dP = do . value row; far - near for rungs ----
    float dp[4 * kWG + MAXK], dpd[MAXK];
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
        f4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (4 * g <= W) acc = row_dot_group(dov, lds0, (s0 - 4 * g) * kRowBytes, swz(s0 - 4 * g));
#pragma unroll
        for (int r = 0; r < 4; ++r) dp[4 * g + r] = acc[r];
    }
    publish<0>();
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            dp[4 * kWG + 2 * k + e] = 0.f;
            dpd[2 * k + e] = 0.f;
        }
        if (k < n_steps) {
            if (k + 1 < n_steps) step(vrs, buf(k + 2), k + 1);
            const f4_t acc = row_dot_group(dov, buf(k + 1), rbase, rsw);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int n = 2 * k + e;
                if (n < n_reach) {
                    const float dd = acc[2 * e + 1] - acc[2 * e];
                    dp[4 * kWG + n] = fmaf(A.off[n].t, dd, acc[2 * e]);
                    dpd[n] = dd;
                }
            }
            publish<0>();
        }
    }

    // ---- softmax gradient; then key window and key step 0 again ----
    float delta = 0.f;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) delta = fmaf(s[y], dp[y], delta);
    // dS = p (dP - delta) / sqrt(D), in place of dP; d(loss)/dt terms
    float dt[MAXK];
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) dp[y] = s[y] * (dp[y] - delta) * A.scale;
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        // dS (q . (k_far - k_near)) / sqrt(D) = (dS / sqrt(D)) sd ln2 sqrt(D) / ... in base 2:
        // sd = (q . dk) log2(e) / sqrt(D), so dS sd ln2 = dS (q . dk) / sqrt(D)
        dt[n] = fmaf(dp[4 * kWG + n] * (kLn2 / A.scale), sd[n], s[4 * kWG + n] * dpd[n]);
    }
    // weights for the key side: term v of key row j = i - delta_v
    if (active) {
        uint32_t* wrow = A.wts + (static_cast<int64_t>(b) * A.Hq + h0 + x) * L * kNV;
#pragma unroll
        for (int d = 0; d < 4 * kWG; ++d)
            if (i - d >= 0) wrow[static_cast<int64_t>(i - d) * kNV + d] = pack_p_ds(s[d], dp[d]);
#pragma unroll
        for (int n = 0; n < MAXK; ++n) {
            if (n < n_reach) {
                const float t = A.off[n].t;
                const int jn = i - A.off[n].a;
                const float pn = s[4 * kWG + n], dn = dp[4 * kWG + n];
                if (jn >= 0) wrow[static_cast<int64_t>(jn) * kNV + 16 + 2 * n] = pack_p_ds(pn - pn * t, dn - dn * t);
                if (jn - 1 >= 0) wrow[static_cast<int64_t>(jn - 1) * kNV + 17 + 2 * n] = pack_p_ds(pn * t, dn * t);
            }
        }
    }
    // (the stores above count in vmcnt: the key blocks are issued after them, so the wait below
    // leaves key step 0 in flight)
    st.window(krs, lds0, jw);
    step(krs, lds1, 0);
    // pass C weights: dS/sqrt(D) times the coefficients, fp16, groups of 4
    uint32_t ww[kWG][2], wo[MAXS][2];
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
        ww[g][0] = pack_h2(dp[4 * g], dp[4 * g + 1]);
        ww[g][1] = pack_h2(dp[4 * g + 2], dp[4 * g + 3]);
    }
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
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
    publish<6>();

    // ---- pass C: dq_rot = sum of weighted key rows (transposing reads of the permuted keys:
    // lane x gets element 4m + x, which is dim 16x + m) ----
    const int pt = 16 * wave + 4 * (pq >> 2) + x;
    const int kt = pq & 3;
    f4_t o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (f4_t){0.f, 0.f, 0.f, 0.f};
    {
        const int sv = pt - kt + W + kWinPad;
#pragma unroll
        for (int g = 0; g < kWG; ++g)
            if (4 * g <= W) row_sum_group(o, ww[g][0], ww[g][1], lds0, (sv - 4 * g) * kRowBytes, swz(sv - 4 * g));
        publish<0>();
    }
    {
        const int sv = (kt < 2) ? pt + 1 - kt : kBlkSlots + pt + 5 - kt;
        const int vbase = sv * kRowBytes, vsw = swz(sv);
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if (k < n_steps) {
                if (k + 1 < n_steps) step(krs, buf(k + 2), k + 1);
                row_sum_group(o, wo[k][0], wo[k][1], buf(k + 1), vbase, vsw);
                if (k + 1 < n_steps) publish<0>();
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- dq: RoPE transposed at position i. Lane x holds dims 16x + m of heads 0..3; the other
    // half of pair (16x + m) mod 32 is in lane x ^ 2 ----
    if (active) {
        const float4* ct = reinterpret_cast<const float4*>(A.cstab) + static_cast<int64_t>(i) * (kPairs / 2) + 8 * (x & 1);
        float2 cs[16];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float4 t = ct[u];
            cs[2 * u] = make_float2(t.x, t.y);
            cs[2 * u + 1] = make_float2(t.z, t.w);
        }
        const float sg = (x < 2) ? 1.f : -1.f;         // x' = x c + y s;  y' = y c - x s
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float other = quad_f<kXor2>(o[m][r]);
                v[m] = fmaf(sg * other, cs[m].y, o[m][r] * cs[m].x);
            }
            bf16_t* drow = static_cast<bf16_t*>(A.dq) + (static_cast<int64_t>(b) * A.Hq + h0 + r) * L * kD +
                           static_cast<int64_t>(i) * kD + 16 * x;
            uint4 lo, hi;
            lo.x = pack_bf2(v[0], v[1]);
            lo.y = pack_bf2(v[2], v[3]);
            lo.z = pack_bf2(v[4], v[5]);
            lo.w = pack_bf2(v[6], v[7]);
            hi.x = pack_bf2(v[8], v[9]);
            hi.y = pack_bf2(v[10], v[11]);
            hi.z = pack_bf2(v[12], v[13]);
            hi.w = pack_bf2(v[14], v[15]);
            *reinterpret_cast<uint4*>(drow) = lo;
            *reinterpret_cast<uint4*>(drow + 8) = hi;
        }
    }

    // ---- d(loss)/dt partial sums of this workgroup, fixed order ----
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        float v = active ? dt[n] : 0.f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[wave][n] = v;
    }
    __syncthreads();
    if (threadIdx.x < static_cast<unsigned>(A.n_off)) {
        float v = 0.f;
        if (threadIdx.x < MAXK) v = ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) + red[3][threadIdx.x];
        A.partial[static_cast<int64_t>(blockIdx.x) * kMaxOff + threadIdx.x] = v;
    }
}

// ------------------------------------------------------------------------------------------------
// bwd_k_dot
// ------------------------------------------------------------------------------------------------
template <int MAXS>
__global__ __launch_bounds__(kNT, 2) void bwd_k_dot_kernel(BwdArgs A) {
    __shared__ __attribute__((aligned(1024))) char lds0[kBufBytes];   // rotated-query blocks
    __shared__ __attribute__((aligned(1024))) char lds1[kBufBytes];   // do blocks

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int pq = lane >> 2, x = lane & 3;
    const int r = 16 * wave + pq;                       // key row of this lane within the tile
    const int L = A.L, W = A.W;
    const int n_tiles = (L + kTile - 1) / kTile;
    int unit, tile;
    unit_tile(blockIdx.x, n_tiles, A.xcd_map, unit, tile);
    const int bg = unit;                                // b * Hkv + g
    const int b = bg / A.Hkv, g = bg % A.Hkv;
    const int j0 = tile * kTile;
    const int j = j0 + r;

    // rungs some key row of the tile receives (query j + a < L): a prefix
    int n_reach = 0;
    for (int n = 0; n < A.n_off; ++n)
        if (j0 + A.off[n].a < L) n_reach = n + 1;
    const int n_steps = (n_reach + 1) >> 1;

    Stager st;
    st.init(lane, wave);
    // key row r's terms: window distance d at slot r + d; rung 2k near at slot r, far at r + 1
    // (block A), rung 2k + 1 near at 72 + r + 2, far at 72 + r + 3 (block B)
    auto step = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int k) {
        st.step(rs, dst, 2 * k < n_reach, j0 + A.off[2 * k].a, 2 * k + 1 < n_reach, j0 + A.off[2 * k + 1].a - 2);
    };
    // transposing reads: lane (p', x) reads for key row rt = 16w + 4 (p' >> 2) + x, term kt = p' & 3
    const int rt = 16 * wave + 4 * (pq >> 2) + x;
    const int kt = pq & 3;
    const int swin = rt + kt;                           // window group g: slot swin + 4g
    const int srung = (kt < 2) ? rt + kt : kBlkSlots + rt + 2 + (kt - 2);
    const int rgbase = srung * kRowBytes, rgsw = swz(srung);

    // validity of a term for key row j: its query q_i = j + delta must exist and read this row
    auto term_ok = [&](int delta, bool interp_near) { return j + delta < L && !(interp_near && j == 0); };

    float dk[16], dv[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        dk[m] = 0.f;
        dv[m] = 0.f;
    }

    for (int hh = 0; hh < A.G; ++hh) {
        const int h = g * A.G + hh;
        const int64_t hrow0 = (static_cast<int64_t>(b) * A.Hq + h) * L;
        const __amdgpu_buffer_rsrc_t qrs = rows_rsrc(A.qrot16, hrow0, L);
        const __amdgpu_buffer_rsrc_t drs = rows_rsrc(A.do16, hrow0, L);
        const uint4* wrow = reinterpret_cast<const uint4*>(A.wts + (hrow0 + (j < L ? j : 0)) * kNV);

        // all of this head's weights for key row j (16-byte loads, issued before the head's first
        // DMA: loads count in vmcnt with the DMAs, in issue order)
        uint4 wl[(4 * kWG + 2 * MAXS * 2) / 4];
#pragma unroll
        for (int u = 0; u < (4 * kWG + 2 * MAXS * 2) / 4; ++u) wl[u] = wrow[u];
        // 4 terms' weights: fp16 ds pairs and fp16 p pairs (masked terms are 0)
        auto weights = [&](int v0, const bool (&ok)[4], uint32_t& ds01, uint32_t& ds23, uint32_t& p01, uint32_t& p23) {
            const uint4 e = wl[v0 >> 2];
            uint32_t w[4] = {e.x, e.y, e.z, e.w};
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] &= (ok[t] && j < L) ? 0xffffffffu : 0u;
            p01 = __builtin_amdgcn_perm(w[1], w[0], 0x05040100u);
            p23 = __builtin_amdgcn_perm(w[3], w[2], 0x05040100u);
            ds01 = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);
            ds23 = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
        };
        // accumulate 4 terms: acc[m] += dot(w01, rows01[4m + x]) + dot(w23, rows23[4m + x]). The 16
        // transposing reads are issued first; each result then passes an empty asm as a 64-bit
        // value before it is split into its two dwords (an optimisation has been seen to fold the
        // second dword of the read onto the first).
        auto sum_terms = [&](float (&acc)[16], uint32_t w01, uint32_t w23, const char* lds, int base, int F) {
            unsigned long long rv[16];
#pragma unroll
            for (int m = 0; m < 16; ++m)
                rv[m] = __builtin_bit_cast(unsigned long long,
                                           tr_read_h4(lds, (base | (((m >> 1) << 4) ^ F)) + 8 * (m & 1)));
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                asm volatile("" : "+v"(rv[m]));
                const uint32_t lo = static_cast<uint32_t>(rv[m]), hi = static_cast<uint32_t>(rv[m] >> 32);
                acc[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w01), __builtin_bit_cast(h2_t, lo), acc[m], false);
                acc[m] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, w23), __builtin_bit_cast(h2_t, hi), acc[m], false);
            }
        };

        // items of this head: window (rotated q, then do), steps (rotated q, then do); an item
        // sits in lds0 (rotated q) or lds1 (do); the next item is issued before each is summed
        // (global loads count in vmcnt with the DMAs, in issue order: weights are loaded before the
        // DMA that must stay in flight while they are used)
        uint32_t wq[kWG][4];                            // window weights (ds01, ds23, p01, p23)
#pragma unroll
        for (int gg = 0; gg < kWG; ++gg) {
            const bool ok[4] = {term_ok(4 * gg, false), term_ok(4 * gg + 1, false), term_ok(4 * gg + 2, false),
                                term_ok(4 * gg + 3, false)};
            weights(4 * gg, ok, wq[gg][0], wq[gg][1], wq[gg][2], wq[gg][3]);
        }
        if (hh == 0) st.window(qrs, lds0, j0);          // later heads: issued at the end of the previous head
        st.window(drs, lds1, j0);
        publish<3>();                                   // the rotated-q window has landed
#pragma unroll
        for (int gg = 0; gg < kWG; ++gg)
            if (4 * gg <= W) sum_terms(dk, wq[gg][0], wq[gg][1], lds0, (swin + 4 * gg) * kRowBytes, swz(swin + 4 * gg));
        publish<0>();                                   // do window landed, lds0 free
        if (n_steps > 0) step(qrs, lds0, 0);
        else if (hh + 1 < A.G) st.window(rows_rsrc(A.qrot16, hrow0 + L, L), lds0, j0);
#pragma unroll
        for (int gg = 0; gg < kWG; ++gg)
            if (4 * gg <= W) sum_terms(dv, wq[gg][2], wq[gg][3], lds1, (swin + 4 * gg) * kRowBytes, swz(swin + 4 * gg));
        publish<0>();
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if (k < n_steps) {
                // rotated-q step k in lds0; its weights, then issue do step k
                uint32_t w4[4];
                {
                    const int n0 = 2 * k, n1 = 2 * k + 1;
                    const bool i0n = n0 < A.n_off && A.off[n0].interp, i1n = n1 < A.n_off && A.off[n1].interp;
                    const int a0 = A.off[n0].a, a1 = A.off[n1].a;
                    const bool ok[4] = {n0 < A.n_off && term_ok(a0, i0n), n0 < A.n_off && term_ok(a0 + 1, false),
                                        n1 < A.n_off && term_ok(a1, i1n), n1 < A.n_off && term_ok(a1 + 1, false)};
                    weights(16 + 4 * k, ok, w4[0], w4[1], w4[2], w4[3]);
                }
                step(drs, lds1, k);
                sum_terms(dk, w4[0], w4[1], lds0, rgbase, rgsw);
                publish<0>();                           // do step k landed, lds0 free
                if (k + 1 < n_steps) step(qrs, lds0, k + 1);
                else if (hh + 1 < A.G) st.window(rows_rsrc(A.qrot16, hrow0 + L, L), lds0, j0);
                sum_terms(dv, w4[2], w4[3], lds1, rgbase, rgsw);
                publish<0>();
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if (j < L) {
        // dk: lane x holds dims 16x + m of dk_rot; RoPE transposed at key position j, the other
        // half of pair (16x + m) mod 32 in lane x ^ 2
        const float4* ct = reinterpret_cast<const float4*>(A.cstab) + static_cast<int64_t>(j) * (kPairs / 2) + 8 * (x & 1);
        const float sg = (x < 2) ? 1.f : -1.f;
        float v[16];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float4 t = ct[u];
            const float o0 = quad_f<kXor2>(dk[2 * u]), o1 = quad_f<kXor2>(dk[2 * u + 1]);
            v[2 * u] = fmaf(sg * o0, t.y, dk[2 * u] * t.x);
            v[2 * u + 1] = fmaf(sg * o1, t.w, dk[2 * u + 1] * t.z);
        }
        const int64_t orow = (static_cast<int64_t>(bg) * L + j) * kD;
        bf16_t* dkr = static_cast<bf16_t*>(A.dk) + orow + 16 * x;
        *reinterpret_cast<uint4*>(dkr) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                                                    pack_bf2(v[6], v[7]));
        *reinterpret_cast<uint4*>(dkr + 8) = make_uint4(pack_bf2(v[8], v[9]), pack_bf2(v[10], v[11]),
                                                        pack_bf2(v[12], v[13]), pack_bf2(v[14], v[15]));
    }
    // dv: lane x holds dims 4m + x; regroup through LDS (lds1 is free) so that lane x writes dims
    // 16x..16x+15
    __syncthreads();
    {
        bf16_t* t = reinterpret_cast<bf16_t*>(lds1) + r * kD;
#pragma unroll
        for (int m = 0; m < 16; ++m) t[4 * m + x] = static_cast<bf16_t>(pack_bf2(dv[m], 0.f) & 0xffffu);
    }
    __syncthreads();
    if (j < L) {
        const uint4* t = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(lds1) + r * kD + 16 * x);
        uint4* dvr = reinterpret_cast<uint4*>(static_cast<bf16_t*>(A.dv) + (static_cast<int64_t>(bg) * L + j) * kD + 16 * x);
        dvr[0] = t[0];
        dvr[1] = t[1];
    }
}

}  // namespace

bool bwd_mfma_supported(const BwdArgs& A) {
    return A.G % 4 == 0 && A.W <= 15 && A.n_off <= 16;
}

hipError_t launch_bwd_mfma(const BwdArgs& A0, bool want_dalpha, int stages, hipStream_t s) {
    BwdArgs A = A0;
    const int64_t n_tiles = (A.L + kTile - 1) / kTile;
    const int64_t q_units = static_cast<int64_t>(A.B) * A.Hkv * (A.G / 4);
    const int64_t k_units = static_cast<int64_t>(A.B) * A.Hkv;
    A.n_wg = static_cast<int32_t>(q_units * n_tiles);
    if (stages & kStageQuery) {
        A.xcd_map = (q_units % 8 == 0) ? 1 : 0;
        hipLaunchKernelGGL((bwd_q_mfma_kernel<8>), dim3(static_cast<unsigned>(q_units * n_tiles)), dim3(kNT), 0, s,
                           A);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & kStageKey) {
        A.xcd_map = (k_units % 8 == 0) ? 1 : 0;
        hipLaunchKernelGGL((bwd_k_dot_kernel<8>), dim3(static_cast<unsigned>(k_units * n_tiles)), dim3(kNT), 0, s,
                           A);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || !want_dalpha) return e;
        return launch_dalpha(A, s);
    }
    return hipSuccess;
}

}  // namespace fibattn
