// Backward pass of Fibonacci-offset sparse attention for gfx950.
//
// Gradients of sum(do * o) through the softmax, the interpolated shifted gather and RoPE
// ("Depth-Staggered Fibonacci Spacing for Sparse Attention", §2 "Attended set": the interpolated
// read is what carries a gradient to alpha; §2 "Per-layer scalar": alpha = 0.5 + sigmoid(theta)).
//
// Three kernels, no atomics (results are bitwise reproducible):
//  * bwd_query: workgroup = (batch, kv head, head chunk, 64 queries), like the forward.
//      pass K1: every score s, and lse = log sum exp s (recomputed here in float32, so the
//               gradients do not inherit the rounding of the forward's lse or o);
//      pass V:  p = exp(s - lse), dP_s = do . val_s, and for interpolated slots
//               g_s = do . (far - near);
//               delta = sum_s p_s dP_s (equal to do . o, but from the float32 probabilities
//               rather than from o rounded to its storage type), dS = p (dP - delta);
//      pass K2: dq_rot += dS key_s / sqrt(D), dt_s = dS (q_rot . (far - near)) / sqrt(D) + p g_s;
//      writes dq (RoPE transposed), the rotated q, p and dS/sqrt(D) per (query, slot), and one
//      fixed-order sum of dt per offset per workgroup.
//  * bwd_key: workgroup = (batch, kv head, 64 key rows). A key row j is read by query j + a of
//      every slot at distance a (weight 1, or 1 - t for the nearer row of an interpolated slot)
//      and by query j + a + 1 of an interpolated slot (weight t): shifted reads again, so dk and
//      dv are gathered, not scattered.
//  * dalpha: one workgroup sums the per-workgroup partials in a fixed order:
//      dalpha = sum_k f_k sum dt_k, dtheta = dalpha * dalpha/dtheta.
#include "fibattn_device.h"

namespace fibattn {

namespace {

constexpr int kPitch = kD + 4;
constexpr int kMaxRows = kTile + kMaxWin;

template <typename T, int NT>
__device__ __forceinline__ void stage_rows(float* buf, const T* base, int j0, int nrows, int L) {
    for (int e = threadIdx.x; e < nrows * (kD / 4); e += NT) {
        const int r = e >> 4, c = e & 15;
        const int j = j0 + r;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j >= 0 && j < L) x = load4<T>(base + static_cast<int64_t>(j) * kD + 4 * c);
        *reinterpret_cast<float4*>(buf + r * kPitch + 4 * c) = x;
    }
}

__device__ __forceinline__ float dot_row(const float (&x)[kD], const float* row) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 k = reinterpret_cast<const float4*>(row)[c];
        a0 = fmaf(x[4 * c + 0], k.x, a0);
        a1 = fmaf(x[4 * c + 1], k.y, a1);
        a2 = fmaf(x[4 * c + 2], k.z, a2);
        a3 = fmaf(x[4 * c + 3], k.w, a3);
    }
    return (a0 + a1) + (a2 + a3);
}

// x . near and x . (far - near)
__device__ __forceinline__ void dot_pair(const float (&x)[kD], const float* near, const float* far,
                                         float& dn, float& dd) {
    float a0 = 0.f, a1 = 0.f, b0 = 0.f, b1 = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 n = reinterpret_cast<const float4*>(near)[c];
        const float4 f = reinterpret_cast<const float4*>(far)[c];
        a0 = fmaf(x[4 * c + 0], n.x, a0);
        a1 = fmaf(x[4 * c + 1], n.y, a1);
        a0 = fmaf(x[4 * c + 2], n.z, a0);
        a1 = fmaf(x[4 * c + 3], n.w, a1);
        b0 = fmaf(x[4 * c + 0], f.x - n.x, b0);
        b1 = fmaf(x[4 * c + 1], f.y - n.y, b1);
        b0 = fmaf(x[4 * c + 2], f.z - n.z, b0);
        b1 = fmaf(x[4 * c + 3], f.w - n.w, b1);
    }
    dn = a0 + a1;
    dd = b0 + b1;
}

__device__ __forceinline__ void axpy_row(float (&o)[kD], float p, const float* row) {
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 v = reinterpret_cast<const float4*>(row)[c];
        o[4 * c + 0] = fmaf(p, v.x, o[4 * c + 0]);
        o[4 * c + 1] = fmaf(p, v.y, o[4 * c + 1]);
        o[4 * c + 2] = fmaf(p, v.z, o[4 * c + 2]);
        o[4 * c + 3] = fmaf(p, v.w, o[4 * c + 3]);
    }
}

__device__ __forceinline__ void axpy_blend(float (&o)[kD], float p, const float* near,
                                           const float* far, float t) {
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 n = reinterpret_cast<const float4*>(near)[c];
        const float4 f = reinterpret_cast<const float4*>(far)[c];
        o[4 * c + 0] = fmaf(p, fmaf(t, f.x - n.x, n.x), o[4 * c + 0]);
        o[4 * c + 1] = fmaf(p, fmaf(t, f.y - n.y, n.y), o[4 * c + 1]);
        o[4 * c + 2] = fmaf(p, fmaf(t, f.z - n.z, n.z), o[4 * c + 2]);
        o[4 * c + 3] = fmaf(p, fmaf(t, f.w - n.w, n.w), o[4 * c + 3]);
    }
}

// Fixed-order sum of v over the workgroup; every thread gets the result. Two barriers.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += red[w];
    return s;
}

// ------------------------------------------------------------------------------------------------
// bwd_query. Per-slot values live in the workspace columns p[bh][slot][i] and dS[bh][slot][i]
// (each thread reads back only what it wrote), so the slot loops need no register arrays.
// ------------------------------------------------------------------------------------------------
template <typename T, int HPB>
__global__ __launch_bounds__(kTile * HPB) void bwd_query_kernel(BwdArgs A) {
    constexpr int NT = kTile * HPB;
    constexpr float kLog2e = 1.44269504088896340736f;
    __shared__ __attribute__((aligned(16))) float buf[kMaxRows * kPitch];
    __shared__ float2 cs_tab[kTile][kPairs];
    __shared__ float red[NT / 64];
    __shared__ float dt_acc[kMaxOff];

    const int p = threadIdx.x / HPB;
    const int hh = threadIdx.x % HPB;
    const int i0 = blockIdx.x * kTile;
    const int n_chunk = A.G / HPB;
    const int g = blockIdx.y / n_chunk;
    const int h = g * A.G + (blockIdx.y % n_chunk) * HPB + hh;
    const int b = blockIdx.z;
    const int i = i0 + p;
    const int L = A.L, W = A.W, S = A.S;
    const bool active = i < L;

    for (int e = threadIdx.x; e < kTile * kPairs; e += NT) {
        const int pp = e / kPairs, m = e % kPairs;
        float c, s;
        rope_cos_sin(i0 + pp, A.fr.hi[m], A.fr.lo[m], c, s);
        cs_tab[pp][m] = make_float2(c, s);
    }
    if (threadIdx.x < kMaxOff) dt_acc[threadIdx.x] = 0.f;
    __syncthreads();

    const int64_t bh = static_cast<int64_t>(b) * A.Hq + h;
    const int64_t qrow = (bh * L + i) * kD;
    const float qs2 = A.scale * kLog2e;
    const int64_t kv_base = (static_cast<int64_t>(b) * A.Hkv + g) * L * kD;
    const float* krot = A.krot + kv_base;
    const T* vsrc = static_cast<const T*>(A.v) + kv_base;
    // this thread's column of the slot tables (only touched when active)
    float* pcol = A.pbuf + bh * S * L + (active ? i : 0);
    float* dcol = A.dsbuf + bh * S * L + (active ? i : 0);

    float x[kD];   // q_rot in the K passes, do in the V pass
    if (active) {
        load_row<T>(static_cast<const T*>(A.q) + qrow, x);
    } else {
#pragma unroll
        for (int e = 0; e < kD; ++e) x[e] = 0.f;
    }
    rope_apply(x, cs_tab[p]);
    if (active) store_row<float>(A.qrot + qrow, x);

    // ---- pass K1: base-2 scores into the p column, running max and sum for lse ----
    constexpr float kNegInf = -__builtin_huge_valf();
    float mx = kNegInf, sm = 0.f;
    auto keep = [&](int slot, float s2) {
        if (!active) return;
        pcol[static_cast<int64_t>(slot) * L] = s2;
        if (s2 > mx) {
            sm = sm * exp2f(mx - s2) + 1.f;
            mx = s2;
        } else if (s2 != kNegInf) {
            sm += exp2f(s2 - mx);
        }
    };
    stage_rows<float, NT>(buf, krot, i0 - W, kTile + W, L);
    __syncthreads();
    for (int d = 0; d <= W; ++d) {
        float s2 = kNegInf;
        if (active && i >= d) s2 = dot_row(x, buf + (p + W - d) * kPitch) * qs2;
        keep(d, s2);
    }
    __syncthreads();
    for (int n = 0; n < A.n_off; ++n) {
        const int a = A.off[n].a;
        const int reach = a + A.off[n].interp;
        float s2 = kNegInf;
        if (i0 + kTile - 1 >= reach) {
            stage_rows<float, NT>(buf, krot, i0 - a - 1, kTile + 1, L);
            __syncthreads();
            const float* near = buf + (p + 1) * kPitch;
            if (active && i >= reach) {
                if (A.off[n].interp) {
                    float dn, dd;
                    dot_pair(x, near, near - kPitch, dn, dd);
                    s2 = fmaf(A.off[n].t, dd, dn) * qs2;
                } else {
                    s2 = dot_row(x, near) * qs2;
                }
            }
            __syncthreads();
        }
        keep(W + 1 + n, s2);
    }
    const float lse2 = active ? mx + log2f(sm) : 0.f;

    // ---- pass V: p = exp(s - lse) (into the p column), dP_s (kept in the dS column), delta,
    // and the p g part of dt ----
    if (active) load_row<T>(static_cast<const T*>(A.dout) + qrow, x);
    float delta = 0.f;
    stage_rows<T, NT>(buf, vsrc, i0 - W, kTile + W, L);
    __syncthreads();
    for (int d = 0; d <= W; ++d) {
        if (!active) continue;
        const float pr = exp2f(pcol[static_cast<int64_t>(d) * L] - lse2);
        pcol[static_cast<int64_t>(d) * L] = pr;
        float dp = 0.f;
        if (pr > 0.f) {
            dp = dot_row(x, buf + (p + W - d) * kPitch);
            delta = fmaf(pr, dp, delta);
        }
        dcol[static_cast<int64_t>(d) * L] = dp;
    }
    __syncthreads();
    for (int n = 0; n < A.n_off; ++n) {
        const int a = A.off[n].a;
        const int reach = a + A.off[n].interp;
        if (i0 + kTile - 1 < reach) {
            if (active) {
                pcol[static_cast<int64_t>(W + 1 + n) * L] = 0.f;
                dcol[static_cast<int64_t>(W + 1 + n) * L] = 0.f;
            }
            continue;
        }
        stage_rows<T, NT>(buf, vsrc, i0 - a - 1, kTile + 1, L);
        __syncthreads();
        const float* near = buf + (p + 1) * kPitch;
        float dp = 0.f, pg = 0.f;
        const float pr = active ? exp2f(pcol[static_cast<int64_t>(W + 1 + n) * L] - lse2) : 0.f;
        if (active) pcol[static_cast<int64_t>(W + 1 + n) * L] = pr;
        if (pr > 0.f) {
            if (A.off[n].interp) {
                float dn, dd;
                dot_pair(x, near, near - kPitch, dn, dd);
                dp = fmaf(A.off[n].t, dd, dn);
                pg = pr * dd;
            } else {
                dp = dot_row(x, near);
            }
            delta = fmaf(pr, dp, delta);
        }
        if (active) dcol[static_cast<int64_t>(W + 1 + n) * L] = dp;
        if (A.off[n].interp) {
            const float sum = block_sum<NT>(pg, red);     // barriers also fence the LDS block
            if (threadIdx.x == 0) dt_acc[n] = sum;
        } else {
            __syncthreads();
        }
    }

    // ---- dS = p (dP - delta) / sqrt(D) ----
    if (active) {
        for (int sl = 0; sl < S; ++sl) {
            const float pr = pcol[static_cast<int64_t>(sl) * L];
            const float dp = dcol[static_cast<int64_t>(sl) * L];
            dcol[static_cast<int64_t>(sl) * L] = pr * (dp - delta) * A.scale;
        }
        load_row<T>(static_cast<const T*>(A.q) + qrow, x);
    }
    rope_apply(x, cs_tab[p]);

    // ---- pass K2: dq_rot and the dS e part of dt ----
    float dqr[kD];
#pragma unroll
    for (int e = 0; e < kD; ++e) dqr[e] = 0.f;
    stage_rows<float, NT>(buf, krot, i0 - W, kTile + W, L);
    __syncthreads();
    for (int d = 0; d <= W; ++d) {
        const float ds = active ? dcol[static_cast<int64_t>(d) * L] : 0.f;
        if (ds != 0.f) axpy_row(dqr, ds, buf + (p + W - d) * kPitch);
    }
    __syncthreads();
    for (int n = 0; n < A.n_off; ++n) {
        const int a = A.off[n].a;
        const int reach = a + A.off[n].interp;
        if (i0 + kTile - 1 < reach) continue;
        stage_rows<float, NT>(buf, krot, i0 - a - 1, kTile + 1, L);
        __syncthreads();
        const float* near = buf + (p + 1) * kPitch;
        const float ds = active ? dcol[static_cast<int64_t>(W + 1 + n) * L] : 0.f;
        float de = 0.f;
        if (A.off[n].interp) {
            if (ds != 0.f) {
                float dn, dd;
                dot_pair(x, near, near - kPitch, dn, dd);
                axpy_blend(dqr, ds, near, near - kPitch, A.off[n].t);
                de = ds * dd;
            }
            const float sum = block_sum<NT>(de, red);
            if (threadIdx.x == 0) dt_acc[n] += sum;
        } else {
            if (ds != 0.f) axpy_row(dqr, ds, near);
            __syncthreads();
        }
    }

    rope_apply_t(dqr, cs_tab[p]);
    if (active) store_row<T>(static_cast<T*>(A.dq) + qrow, dqr);

    __syncthreads();
    if (threadIdx.x < A.n_off) {
        const int64_t wg = (static_cast<int64_t>(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        A.partial[wg * kMaxOff + threadIdx.x] = dt_acc[threadIdx.x];
    }
}

// ------------------------------------------------------------------------------------------------
// bwd_key: thread = (key row r of the tile, head hh of the chunk); heads are summed in LDS.
// ------------------------------------------------------------------------------------------------
template <typename T, int HPB>
__global__ __launch_bounds__(kTile * HPB) void bwd_key_kernel(BwdArgs A) {
    constexpr int NT = kTile * HPB;
    __shared__ float2 cs_tab[kTile][kPairs];
    __shared__ float acc[kTile][2 * kD + 1];

    const int r = threadIdx.x % kTile;    // rows contiguous across lanes: coalesced p/dS reads
    const int hh = threadIdx.x / kTile;
    const int j0 = blockIdx.x * kTile;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int j = j0 + r;
    const int L = A.L, W = A.W, S = A.S;
    const bool active = j < L;

    for (int e = threadIdx.x; e < kTile * kPairs; e += NT) {
        const int pp = e / kPairs, m = e % kPairs;
        float c, s;
        rope_cos_sin(j0 + pp, A.fr.hi[m], A.fr.lo[m], c, s);
        cs_tab[pp][m] = make_float2(c, s);
    }

    float dk[kD], dv[kD];
#pragma unroll
    for (int e = 0; e < kD; ++e) {
        dk[e] = 0.f;
        dv[e] = 0.f;
    }

    if (active) {
        for (int c = 0; c < A.G / HPB; ++c) {
            const int h = g * A.G + c * HPB + hh;
            const int64_t bh = static_cast<int64_t>(b) * A.Hq + h;
            const float* qrot = A.qrot + bh * L * kD;
            const T* dout = static_cast<const T*>(A.dout) + bh * L * kD;
            const float* pb = A.pbuf + bh * S * L;
            const float* db = A.dsbuf + bh * S * L;
            // one (query, slot, weight) term
            auto term = [&](int qi, int slot, float w) {
                if (qi >= L) return;
                const int64_t idx = static_cast<int64_t>(slot) * L + qi;
                const float ds = db[idx] * w, pr = pb[idx] * w;
                if (ds == 0.f && pr == 0.f) return;
                const float* qr = qrot + static_cast<int64_t>(qi) * kD;
                const T* dr = dout + static_cast<int64_t>(qi) * kD;
#pragma unroll
                for (int c = 0; c < kD / 4; ++c) {
                    const float4 a = load4<float>(qr + 4 * c);
                    const float4 u = load4<T>(dr + 4 * c);
                    dk[4 * c + 0] = fmaf(ds, a.x, dk[4 * c + 0]);
                    dk[4 * c + 1] = fmaf(ds, a.y, dk[4 * c + 1]);
                    dk[4 * c + 2] = fmaf(ds, a.z, dk[4 * c + 2]);
                    dk[4 * c + 3] = fmaf(ds, a.w, dk[4 * c + 3]);
                    dv[4 * c + 0] = fmaf(pr, u.x, dv[4 * c + 0]);
                    dv[4 * c + 1] = fmaf(pr, u.y, dv[4 * c + 1]);
                    dv[4 * c + 2] = fmaf(pr, u.z, dv[4 * c + 2]);
                    dv[4 * c + 3] = fmaf(pr, u.w, dv[4 * c + 3]);
                }
            };
            for (int d = 0; d <= W; ++d) term(j + d, d, 1.f);
            for (int n = 0; n < A.n_off; ++n) {
                const int a = A.off[n].a;
                const int slot = W + 1 + n;
                if (A.off[n].interp) {
                    const float t = A.off[n].t;
                    term(j + a, slot, 1.f - t);
                    term(j + a + 1, slot, t);
                } else {
                    term(j + a, slot, 1.f);
                }
            }
        }
    }

    // sum the HPB heads of the chunk in LDS, one head at a time, into head 0's registers
    for (int u = 1; u < HPB; ++u) {
        __syncthreads();
        if (hh == u) {
#pragma unroll
            for (int e = 0; e < kD; ++e) {
                acc[r][e] = dk[e];
                acc[r][kD + e] = dv[e];
            }
        }
        __syncthreads();
        if (hh == 0) {
#pragma unroll
            for (int e = 0; e < kD; ++e) {
                dk[e] += acc[r][e];
                dv[e] += acc[r][kD + e];
            }
        }
    }
    __syncthreads();
    if (hh == 0 && active) {
        rope_apply_t(dk, cs_tab[r]);
        const int64_t row = ((static_cast<int64_t>(b) * A.Hkv + g) * L + j) * kD;
        store_row<T>(static_cast<T*>(A.dk) + row, dk);
        store_row<T>(static_cast<T*>(A.dv) + row, dv);
    }
}

// ------------------------------------------------------------------------------------------------
// dalpha: sum per offset over workgroups in a fixed order (double), weight by f_k. Thread t sums
// column t % kMaxOff over workgroups t / kMaxOff, + kDaRows, ...: the loads of all offsets are in
// flight together (consecutive threads read one workgroup's row), then a tree over the rows.
// ------------------------------------------------------------------------------------------------
constexpr int kDaThreads = 1024, kDaRows = kDaThreads / kMaxOff;
__global__ __launch_bounds__(kDaThreads) void dalpha_kernel(BwdArgs A) {
    __shared__ double red[kDaThreads];
    const int n = threadIdx.x % kMaxOff, r = threadIdx.x / kMaxOff;
    bool use = false;                                   // interpolated kept rung (uniform loop: no
    for (int k = 0; k < A.n_off; ++k)                   // per-lane indexing of the argument block)
        if (k == n && A.off[k].interp) use = true;
    double s = 0.0;
    if (use) {
#pragma unroll 4
        for (int w = r; w < A.n_wg; w += kDaRows) s += A.partial[static_cast<int64_t>(w) * kMaxOff + n];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int stride = kDaRows / 2; stride > 0; stride >>= 1) {
        if (r < stride) red[threadIdx.x] += red[threadIdx.x + stride * kMaxOff];
        __syncthreads();
    }
    double acc = 0.0;
    for (int k = 0; k < A.n_off; ++k)
        if (A.off[k].interp) acc += static_cast<double>(A.off[k].f) * red[k];
    if (threadIdx.x == 0) {
        if (A.dalpha != nullptr) A.dalpha[0] = static_cast<float>(acc);
        if (A.dtheta != nullptr) A.dtheta[0] = static_cast<float>(acc * static_cast<double>(A.dalpha_dtheta));
    }
}

template <typename T, int HPB>
void launch_bwd_heads(const BwdArgs& A, bool want_dalpha, int stages, hipStream_t s) {
    const int tiles = (A.L + kTile - 1) / kTile;
    if (stages & kStageQuery)
        hipLaunchKernelGGL((bwd_query_kernel<T, HPB>), dim3(tiles, A.Hkv * (A.G / HPB), A.B), dim3(kTile * HPB), 0,
                           s, A);
    if (stages & kStageKey) {
        hipLaunchKernelGGL((bwd_key_kernel<T, HPB>), dim3(tiles, A.Hkv, A.B), dim3(kTile * HPB), 0, s, A);
        if (want_dalpha) hipLaunchKernelGGL(dalpha_kernel, dim3(1), dim3(kDaThreads), 0, s, A);
    }
}

template <typename T>
hipError_t launch_bwd_typed(const BwdArgs& A, bool want_dalpha, int stages, hipStream_t s) {
    const int hpb = (A.G % 4 == 0) ? 4 : (A.G % 2 == 0) ? 2 : 1;
    if (hpb == 4) launch_bwd_heads<T, 4>(A, want_dalpha, stages, s);
    else if (hpb == 2) launch_bwd_heads<T, 2>(A, want_dalpha, stages, s);
    else launch_bwd_heads<T, 1>(A, want_dalpha, stages, s);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dalpha(const BwdArgs& A, hipStream_t s) {
    hipLaunchKernelGGL(dalpha_kernel, dim3(1), dim3(kDaThreads), 0, s, A);
    return hipGetLastError();
}

namespace {

}  // namespace

int bwd_query_workgroups(int B, int L, int Hkv, int G) {
    const int hpb = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    return ((L + kTile - 1) / kTile) * Hkv * (G / hpb) * B;
}

hipError_t launch_bwd(int dtype, const BwdArgs& A, bool want_dalpha, int stages, hipStream_t s) {
    return dtype == 0 ? launch_bwd_typed<float>(A, want_dalpha, stages, s)
                      : launch_bwd_typed<bf16_t>(A, want_dalpha, stages, s);
}

}  // namespace fibattn
