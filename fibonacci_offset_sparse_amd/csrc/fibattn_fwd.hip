// Forward pass of Fibonacci-offset sparse attention for gfx950.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv
// 2606.28560): §2 "Attended set" defines the window, the scaled offsets, the interpolated
// shifted gather and RoPE before the gather.
//
// Two kernels:
//  * rope_keys: every key row rotated once at its own position, float32, into the workspace
//    (float32 storage; bf16 storage uses prep_kv16 in fibattn_fwd_mfma.hip).
//  * fwd_attend: the general kernel, used for float32 storage and for shapes outside the fast
//    bf16 kernel (fwd_mfma in fibattn_fwd_mfma.hip). One workgroup per (batch, key-value head, group of query heads, 64 query
//    positions). The offsets are shared by all queries, so the rows one slot needs for the
//    whole tile form one contiguous block: the window block [i0 - W, i0 + 64) and, per offset,
//    [i0 - a - 1, i0 + 64 - a). Each block is staged in LDS by coalesced loads and read by the
//    4 query heads of the key-value head (GQA). Pass 1 stages key blocks and keeps every score
//    in registers; the softmax is then exact (no running rescale); pass 2 stages the value
//    blocks and accumulates P.V.
#include <type_traits>

#include "fibattn_device.h"

namespace fibattn {

namespace {

constexpr int kPitch = kD + 4;                    // LDS row pitch in floats (16-byte aligned)
constexpr int kMaxRows = kTile + kMaxWin;         // window block rows (64 + W <= 95)

// ------------------------------------------------------------------------------------------------
// rope_keys: thread = (row, 4 RoPE pairs), 8 threads per row, all rows in parallel.
// ------------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rope_keys_kernel(RopeKeysArgs A) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int quad = static_cast<int>(gid & 7);                  // pairs 4*quad .. 4*quad+3
    const int64_t row_id = gid >> 3;
    if (row_id >= static_cast<int64_t>(A.n_bh) * A.L) return;
    const int j = static_cast<int>(row_id % A.L);
    const int64_t row = row_id * kD;
    const T* src = static_cast<const T*>(A.k);
    const float4 x1 = load4<T>(src + row + 4 * quad);
    const float4 x2 = load4<T>(src + row + kPairs + 4 * quad);
    const float a[4] = {x1.x, x1.y, x1.z, x1.w};
    const float b[4] = {x2.x, x2.y, x2.z, x2.w};
    float r1[4], r2[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float c, s;
        rope_cos_sin(j, A.fr.hi[4 * quad + u], A.fr.lo[4 * quad + u], c, s);
        r1[u] = a[u] * c - b[u] * s;
        r2[u] = b[u] * c + a[u] * s;
    }
    store4<float>(A.krot + row + 4 * quad, make_float4(r1[0], r1[1], r1[2], r1[3]));
    store4<float>(A.krot + row + kPairs + 4 * quad, make_float4(r2[0], r2[1], r2[2], r2[3]));
}

// ------------------------------------------------------------------------------------------------
// fwd_attend
// ------------------------------------------------------------------------------------------------

// Copy rows [j0, j0 + nrows) of one (batch, head) into LDS as float; rows outside [0, L) are
// zero-filled and never read from memory.
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

// Rows [j0, j0 + nrows) of the caller's bf16 keys into LDS as float32, each rotated at its own
// position (cos/sin from the table): the general kernel's bf16 path reads the caller's rows, so
// that no value leaves the range it can hold. Thread item e: row e / 8, RoPE pairs 4c .. 4c + 3
// (c = e % 8), i.e. dims 4c .. 4c + 3 and 32 + 4c .. 32 + 4c + 3.
template <int NT>
__device__ __forceinline__ void stage_rows_rot(float* buf, const bf16_t* base, const float* cstab, int j0, int nrows,
                                               int L) {
    for (int e = threadIdx.x; e < nrows * 8; e += NT) {
        const int r = e >> 3, c = e & 7;
        const int j = j0 + r;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f), y = x;
        if (j >= 0 && j < L) {
            const float4 a = load4<bf16_t>(base + static_cast<int64_t>(j) * kD + 4 * c);
            const float4 b = load4<bf16_t>(base + static_cast<int64_t>(j) * kD + kPairs + 4 * c);
            const float4* cs = reinterpret_cast<const float4*>(cstab + static_cast<int64_t>(j) * 2 * kPairs + 8 * c);
            const float4 t0 = cs[0], t1 = cs[1];         // (cos, sin) of pairs 4c .. 4c + 3
            x = make_float4(a.x * t0.x - b.x * t0.y, a.y * t0.z - b.y * t0.w, a.z * t1.x - b.z * t1.y,
                            a.w * t1.z - b.w * t1.w);
            y = make_float4(b.x * t0.x + a.x * t0.y, b.y * t0.z + a.y * t0.w, b.z * t1.x + a.z * t1.y,
                            b.w * t1.z + a.w * t1.w);
        }
        *reinterpret_cast<float4*>(buf + r * kPitch + 4 * c) = x;
        *reinterpret_cast<float4*>(buf + r * kPitch + kPairs + 4 * c) = y;
    }
}

__device__ __forceinline__ float dot_row(const float (&q)[kD], const float* row) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 k = reinterpret_cast<const float4*>(row)[c];
        a0 = fmaf(q[4 * c + 0], k.x, a0);
        a1 = fmaf(q[4 * c + 1], k.y, a1);
        a2 = fmaf(q[4 * c + 2], k.z, a2);
        a3 = fmaf(q[4 * c + 3], k.w, a3);
    }
    return (a0 + a1) + (a2 + a3);
}

// q . (near + t (far - near))
__device__ __forceinline__ float dot_blend(const float (&q)[kD], const float* near,
                                           const float* far, float t) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 4; ++c) {
        const float4 n = reinterpret_cast<const float4*>(near)[c];
        const float4 f = reinterpret_cast<const float4*>(far)[c];
        a0 = fmaf(q[4 * c + 0], fmaf(t, f.x - n.x, n.x), a0);
        a1 = fmaf(q[4 * c + 1], fmaf(t, f.y - n.y, n.y), a1);
        a2 = fmaf(q[4 * c + 2], fmaf(t, f.z - n.z, n.z), a2);
        a3 = fmaf(q[4 * c + 3], fmaf(t, f.w - n.w, n.w), a3);
    }
    return (a0 + a1) + (a2 + a3);
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

// The general kernel: any GQA group, W <= 31, up to 32 offsets, float32 arithmetic on staged
// rows. T is the storage type of q and o; KT and VT are the element types of the staged keys and
// values: float32 rotated keys and the float32 input for float32 storage; for bf16 storage the
// caller's bf16 keys (rotated as they are staged, from the cos/sin table) and values.
// HPB query heads per workgroup (the heads of one key-value head, or a chunk of them).
// Thread t: position p = t / HPB of the tile, head h = t % HPB of the chunk, so the HPB heads
// of one position sit in adjacent lanes and read the same LDS row.
template <typename T, typename KT, typename VT, int HPB>
__global__ __launch_bounds__(kTile * HPB) void fwd_attend_kernel(FwdArgs A) {
    constexpr int NT = kTile * HPB;
    constexpr float kNegInf = -__builtin_huge_valf();
    __shared__ __attribute__((aligned(16))) float buf[kMaxRows * kPitch];
    __shared__ float2 cs_tab[kTile][kPairs];

    const int p = threadIdx.x / HPB;
    const int hh = threadIdx.x % HPB;
    const int i0 = blockIdx.x * kTile;
    const int n_chunk = A.G / HPB;
    const int g = blockIdx.y / n_chunk;
    const int h = g * A.G + (blockIdx.y % n_chunk) * HPB + hh;
    const int b = blockIdx.z;
    const int i = i0 + p;
    const int L = A.L, W = A.W;
    const bool active = i < L;

    for (int e = threadIdx.x; e < kTile * kPairs; e += NT) {
        const int pp = e / kPairs, m = e % kPairs;
        float c, s;
        rope_cos_sin(i0 + pp, A.fr.hi[m], A.fr.lo[m], c, s);
        cs_tab[pp][m] = make_float2(c, s);
    }
    __syncthreads();

    const int64_t qrow = ((static_cast<int64_t>(b) * A.Hq + h) * L + i) * kD;
    float q[kD];
    if (active) {
        load_row<T>(static_cast<const T*>(A.q) + qrow, q);
    } else {
#pragma unroll
        for (int e = 0; e < kD; ++e) q[e] = 0.f;
    }
    rope_apply(q, cs_tab[p]);
#pragma unroll
    for (int e = 0; e < kD; ++e) q[e] *= A.qscale;

    const int64_t kv_base = (static_cast<int64_t>(b) * A.Hkv + g) * L * kD;
    const KT* krot = static_cast<const KT*>(A.kstage) + kv_base;
    const VT* vsrc = static_cast<const VT*>(A.vstage) + kv_base;

    // keys: float32 rotated (float32 storage), or the caller's bf16 rows rotated as staged
    auto stage_keys = [&](int j0, int nrows) {
        if constexpr (std::is_same<KT, bf16_t>::value)
            stage_rows_rot<NT>(buf, krot, A.cstab, j0, nrows, L);
        else
            stage_rows<KT, NT>(buf, krot, j0, nrows, L);
    };

    // ---- pass 1: scores (base 2), window then offsets ----
    float sw[kMaxWin], so[kMaxOff];
    stage_keys(i0 - W, kTile + W);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < kMaxWin; ++d) {
        sw[d] = kNegInf;
        if (d <= W && active && i >= d) sw[d] = dot_row(q, buf + (p + W - d) * kPitch);
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) {
        so[n] = kNegInf;
        if (n < A.n_off) {
            const int a = A.off[n].a;
            const int reach = a + A.off[n].interp;
            if (i0 + kTile - 1 >= reach) {                     // some query of the tile reads it
                stage_keys(i0 - a - 1, kTile + 1);
                __syncthreads();
                const float* near = buf + (p + 1) * kPitch;
                if (active && i >= reach)
                    so[n] = A.off[n].interp ? dot_blend(q, near, near - kPitch, A.off[n].t)
                                            : dot_row(q, near);
                __syncthreads();
            }
        }
    }

    // ---- exact softmax over the slots ----
    float m = kNegInf;
#pragma unroll
    for (int d = 0; d < kMaxWin; ++d) m = fmaxf(m, sw[d]);
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) m = fmaxf(m, so[n]);
    if (!active) m = 0.f;
    float l = 0.f;
#pragma unroll
    for (int d = 0; d < kMaxWin; ++d) {
        sw[d] = exp2f(sw[d] - m);
        l += sw[d];
    }
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) {
        so[n] = exp2f(so[n] - m);
        l += so[n];
    }

    // ---- pass 2: P.V ----
    float o[kD];
#pragma unroll
    for (int e = 0; e < kD; ++e) o[e] = 0.f;
    stage_rows<VT, NT>(buf, vsrc, i0 - W, kTile + W, L);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < kMaxWin; ++d)
        if (d <= W && sw[d] > 0.f) axpy_row(o, sw[d], buf + (p + W - d) * kPitch);
    __syncthreads();
#pragma unroll
    for (int n = 0; n < kMaxOff; ++n) {
        if (n < A.n_off) {
            const int a = A.off[n].a;
            const int reach = a + A.off[n].interp;
            if (i0 + kTile - 1 >= reach) {
                stage_rows<VT, NT>(buf, vsrc, i0 - a - 1, kTile + 1, L);
                __syncthreads();
                const float* near = buf + (p + 1) * kPitch;
                if (so[n] > 0.f) {
                    if (A.off[n].interp)
                        axpy_blend(o, so[n], near, near - kPitch, A.off[n].t);
                    else
                        axpy_row(o, so[n], near);
                }
                __syncthreads();
            }
        }
    }

    if (active) {
        const float inv = 1.0f / l;
#pragma unroll
        for (int e = 0; e < kD; ++e) o[e] *= inv;
        store_row<T>(static_cast<T*>(A.o) + qrow, o);
        if (A.lse != nullptr)
            A.lse[(static_cast<int64_t>(b) * A.Hq + h) * L + i] = (m + log2f(l)) * 0.69314718055994530942f;
    }
}

template <typename T, typename KT, typename VT>
hipError_t launch_fwd_typed(const FwdArgs& A, hipStream_t s) {
    const int hpb = (A.G % 4 == 0) ? 4 : (A.G % 2 == 0) ? 2 : 1;
    dim3 grid((A.L + kTile - 1) / kTile, A.Hkv * (A.G / hpb), A.B);
    if (hpb == 4)
        hipLaunchKernelGGL((fwd_attend_kernel<T, KT, VT, 4>), grid, dim3(kTile * 4), 0, s, A);
    else if (hpb == 2)
        hipLaunchKernelGGL((fwd_attend_kernel<T, KT, VT, 2>), grid, dim3(kTile * 2), 0, s, A);
    else
        hipLaunchKernelGGL((fwd_attend_kernel<T, KT, VT, 1>), grid, dim3(kTile), 0, s, A);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_keys(int dtype, const RopeKeysArgs& A, hipStream_t s) {
    const int64_t threads = static_cast<int64_t>(A.n_bh) * A.L * 8;
    const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
    if (dtype == 0)
        hipLaunchKernelGGL((rope_keys_kernel<float>), dim3(blocks), dim3(256), 0, s, A);
    else
        hipLaunchKernelGGL((rope_keys_kernel<bf16_t>), dim3(blocks), dim3(256), 0, s, A);
    return hipGetLastError();
}

hipError_t launch_fwd_attend(int dtype, const FwdArgs& A, hipStream_t s) {
    if (dtype == 0) return launch_fwd_typed<float, float, float>(A, s);
    if (fwd_mfma_supported(A)) return launch_fwd_mfma(A, s);
    // the caller's rows, keys rotated as they are staged: any finite bf16 input
    FwdArgs B = A;
    B.kstage = A.k;
    B.vstage = A.v;
    return launch_fwd_typed<bf16_t, bf16_t, bf16_t>(B, s);
}

}  // namespace fibattn
