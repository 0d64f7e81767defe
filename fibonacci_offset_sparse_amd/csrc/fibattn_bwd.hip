// Backward pass of Fibonacci-offset sparse attention for gfx950.
//
// Gradients of sum(do * o) through the softmax, the interpolated shifted gather and RoPE
// ("Depth-Staggered Fibonacci Spacing for Sparse Attention", §2 "Attended set": the interpolated
// read is what carries a gradient to alpha; §2 "Per-layer scalar": alpha = 0.5 + sigmoid(theta)).
//
// Three kernels, no atomics (results are bitwise reproducible):
//  * bwd_query: workgroup = (batch, kv head, head chunk, 64 queries), like the forward.
//      pass V: dP_s = do . val_s, and for interpolated slots g_s = do . (far - near);
//      pass K: s -> p = exp(s - lse), dS = p (dP - delta) with delta = do . o,
//              dq_rot += dS key_s / sqrt(D), dt_s = dS (q_rot . (far - near)) / sqrt(D) + p g_s;
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

// ------------------------------------------------------------------------------------------------
// bwd_query
// ------------------------------------------------------------------------------------------------
template <typename T, int HPB>
__global__ __launch_bounds__(kTile * HPB) void bwd_query_kernel(BwdArgs A) {
    constexpr int NT = kTile * HPB;
    constexpr float kLog2e = 1.44269504088896340736f;
    __shared__ __attribute__((aligned(16))) float buf[kMaxRows * kPitch];
    __shared__ float2 cs_tab[kTile][kPairs];
    __shared__ float red[NT / 64][kMaxOff];

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
    __syncthreads();

    const int64_t bh = static_cast<int64_t>(b) * A.Hq + h;
    const int64_t qrow = (bh * L + i) * kD;
    float x[kD];   // do during pass V, q_rot during pass K
    float lse2 = 0.f, delta = 0.f;
    if (active) {
        float ov[kD];
        load_row<T>(static_cast<const T*>(A.o) + qrow, ov);
        load_row<T>(static_cast<const T*>(A.dout) + qrow, x);
#pragma unroll
        for (int e = 0; e < kD; ++e) delta = fmaf(x[e], ov[e], delta);
        lse2 = A.lse[bh * L + i] * kLog2e;
    } else {
#pragma unroll
        for (int e = 0; e < kD; ++e) x[e] = 0.f;
    }

    const int64_t kv_base = (static_cast<int64_t>(b) * A.Hkv + g) * L * kD;
    const float* krot = A.krot + kv_base;
    const T* vsrc = static_cast<const T*>(A.v) + kv_base;

    // ---- pass V ----
    float dpw[kMaxWin], dpo[kMaxOff], gvo[kMaxOff];
    stage_rows<T, NT>(buf, vsrc, i0 - W, kTile + W, L);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < kMaxWin; ++d) {
        dpw[d] = 0.f;
        if (d <= W && active && i >= d) dpw[d] = dot_row(x, buf + (p + W - d) * kPitch);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) {
        dpo[n] = 0.f;
        gvo[n] = 0.f;
        if (n < A.n_off) {
            const int a = A.off[n].a;
            const int reach = a + A.off[n].interp;
            if (i0 + kTile - 1 >= reach) {
                stage_rows<T, NT>(buf, vsrc, i0 - a - 1, kTile + 1, L);
                __syncthreads();
                const float* near = buf + (p + 1) * kPitch;
                if (active && i >= reach) {
                    if (A.off[n].interp) {
                        float dn, dd;
                        dot_pair(x, near, near - kPitch, dn, dd);
                        dpo[n] = fmaf(A.off[n].t, dd, dn);
                        gvo[n] = dd;
                    } else {
                        dpo[n] = dot_row(x, near);
                    }
                }
                __syncthreads();
            }
        }
    }

    // ---- q_rot ----
    if (active) {
        load_row<T>(static_cast<const T*>(A.q) + qrow, x);
    } else {
#pragma unroll
        for (int e = 0; e < kD; ++e) x[e] = 0.f;
    }
    rope_apply(x, cs_tab[p]);
    if (active) store_row<float>(A.qrot + qrow, x);

    // ---- pass K ----
    const float qs2 = A.scale * kLog2e;
    float dqr[kD];
#pragma unroll
    for (int e = 0; e < kD; ++e) dqr[e] = 0.f;
    float dto[kMaxOff];
    float* pcol = A.pbuf + bh * S * L + i;
    float* dcol = A.dsbuf + bh * S * L + i;

    stage_rows<float, NT>(buf, krot, i0 - W, kTile + W, L);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < kMaxWin; ++d) {
        if (d <= W) {
            float pr = 0.f, ds = 0.f;
            if (active && i >= d) {
                const float* row = buf + (p + W - d) * kPitch;
                const float s2 = dot_row(x, row) * qs2;
                pr = exp2f(s2 - lse2);
                ds = pr * (dpw[d] - delta) * A.scale;
                axpy_row(dqr, ds, row);
            }
            if (active) {
                pcol[static_cast<int64_t>(d) * L] = pr;
                dcol[static_cast<int64_t>(d) * L] = ds;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) {
        dto[n] = 0.f;
        if (n < A.n_off) {
            const int a = A.off[n].a;
            const int reach = a + A.off[n].interp;
            const int slot = W + 1 + n;
            float pr = 0.f, ds = 0.f;
            if (i0 + kTile - 1 >= reach) {
                stage_rows<float, NT>(buf, krot, i0 - a - 1, kTile + 1, L);
                __syncthreads();
                const float* near = buf + (p + 1) * kPitch;
                if (active && i >= reach) {
                    if (A.off[n].interp) {
                        const float t = A.off[n].t;
                        float dn, dd;
                        dot_pair(x, near, near - kPitch, dn, dd);
                        const float s2 = fmaf(t, dd, dn) * qs2;
                        pr = exp2f(s2 - lse2);
                        ds = pr * (dpo[n] - delta) * A.scale;
                        axpy_blend(dqr, ds, near, near - kPitch, t);
                        dto[n] = fmaf(ds, dd, pr * gvo[n]);
                    } else {
                        const float s2 = dot_row(x, near) * qs2;
                        pr = exp2f(s2 - lse2);
                        ds = pr * (dpo[n] - delta) * A.scale;
                        axpy_row(dqr, ds, near);
                    }
                }
                __syncthreads();
            }
            if (active) {
                pcol[static_cast<int64_t>(slot) * L] = pr;
                dcol[static_cast<int64_t>(slot) * L] = ds;
            }
        }
    }

    rope_apply_t(dqr, cs_tab[p]);
    if (active) store_row<T>(static_cast<T*>(A.dq) + qrow, dqr);

    // ---- fixed-order workgroup sums of dt per offset ----
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) {
        if (n < A.n_off) {
            float v = dto[n];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wave][n] = v;
        }
    }
    __syncthreads();
    if (threadIdx.x < A.n_off) {
        float s = 0.f;
        for (int w = 0; w < NT / 64; ++w) s += red[w][threadIdx.x];
        const int64_t wg = (static_cast<int64_t>(blockIdx.z) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
        A.partial[wg * kMaxOff + threadIdx.x] = s;
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
                float xr[kD];
                load_row<float>(qrot + static_cast<int64_t>(qi) * kD, xr);
#pragma unroll
                for (int e = 0; e < kD; ++e) dk[e] = fmaf(ds, xr[e], dk[e]);
                load_row<T>(dout + static_cast<int64_t>(qi) * kD, xr);
#pragma unroll
                for (int e = 0; e < kD; ++e) dv[e] = fmaf(pr, xr[e], dv[e]);
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
// dalpha: sum per offset over workgroups in a fixed order (double), weight by f_k.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dalpha_kernel(BwdArgs A) {
    __shared__ double red[256];
    double acc = 0.0;
    for (int n = 0; n < A.n_off; ++n) {
        if (!A.off[n].interp) continue;
        double s = 0.0;
        for (int w = threadIdx.x; w < A.n_wg; w += 256) s += A.partial[static_cast<int64_t>(w) * kMaxOff + n];
        red[threadIdx.x] = s;
        __syncthreads();
        for (int stride = 128; stride > 0; stride >>= 1) {
            if (threadIdx.x < stride) red[threadIdx.x] += red[threadIdx.x + stride];
            __syncthreads();
        }
        acc += static_cast<double>(A.off[n].f) * red[0];
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        if (A.dalpha != nullptr) A.dalpha[0] = static_cast<float>(acc);
        if (A.dtheta != nullptr) A.dtheta[0] = static_cast<float>(acc * static_cast<double>(A.dalpha_dtheta));
    }
}

template <typename T>
hipError_t launch_bwd_typed(const BwdArgs& A, bool want_dalpha, hipStream_t s) {
    const int hpb = (A.G % 4 == 0) ? 4 : (A.G % 2 == 0) ? 2 : 1;
    const int tiles = (A.L + kTile - 1) / kTile;
    dim3 gq(tiles, A.Hkv * (A.G / hpb), A.B);
    dim3 gk(tiles, A.Hkv, A.B);
    if (hpb == 4) {
        hipLaunchKernelGGL((bwd_query_kernel<T, 4>), gq, dim3(kTile * 4), 0, s, A);
        hipLaunchKernelGGL((bwd_key_kernel<T, 4>), gk, dim3(kTile * 4), 0, s, A);
    } else if (hpb == 2) {
        hipLaunchKernelGGL((bwd_query_kernel<T, 2>), gq, dim3(kTile * 2), 0, s, A);
        hipLaunchKernelGGL((bwd_key_kernel<T, 2>), gk, dim3(kTile * 2), 0, s, A);
    } else {
        hipLaunchKernelGGL((bwd_query_kernel<T, 1>), gq, dim3(kTile), 0, s, A);
        hipLaunchKernelGGL((bwd_key_kernel<T, 1>), gk, dim3(kTile), 0, s, A);
    }
    if (want_dalpha) hipLaunchKernelGGL(dalpha_kernel, dim3(1), dim3(256), 0, s, A);
    return hipGetLastError();
}

}  // namespace

int bwd_query_workgroups(int B, int L, int Hkv, int G) {
    const int hpb = (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
    return ((L + kTile - 1) / kTile) * Hkv * (G / hpb) * B;
}

hipError_t launch_bwd(int dtype, const BwdArgs& A, bool want_dalpha, hipStream_t s) {
    return dtype == 0 ? launch_bwd_typed<float>(A, want_dalpha, s)
                      : launch_bwd_typed<bf16_t>(A, want_dalpha, s);
}

}  // namespace fibattn
