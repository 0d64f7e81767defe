// Forward attention for bfloat16 storage on gfx950: the fast kernel.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv
// 2606.28560), §2 "Attended set": window distances 0..W plus one slot per rung at distance
// d = alpha f, read by linear interpolation between rows i - floor(d) and i - floor(d) - 1, with
// RoPE applied before the gather. Offsets are shared by all queries, so for a tile of 64 queries
// each slot reads one contiguous block of rows.
//
// Inputs come from prep_kv16: keys rotated at their positions and values, both as fp16 rows of
// 128 bytes. A workgroup owns (batch b, key-value head g, 4 query heads, 64 positions) and runs
// 256 lanes as quads: lane 4p + c holds position p and the 16 dims {8c..8c+7, 32+8c..32+8c+7} of
// all 4 query heads (both halves of RoPE pairs 8c..8c+7 stay in one lane). Every staged K/V row
// is read from LDS once per slot, by the 4 lanes of its position, and used for all 4 heads.
//
//  * QK: per head 8 v_dot2_f32_f16 over the lane's 16 dims (fp16 products are exact in fp32,
//    accumulation is fp32), then a 3-step DPP reduce-scatter leaves lane c with head c's score.
//    Register slot k of a lane holds head c ^ k, so the reduction needs no selects.
//  * Interpolated keys are blended in registers with packed fp16 (near + t (far - near)).
//  * Softmax is exact: all scores of the lane's head stay in registers (base-2 exponent).
//  * PV: values enter as pairs of rows with a pair of weights, one v_dot2_f32_f16 per dim and
//    head: window slots d, d + 1 (adjacent rows); an interpolated slot is its own pair
//    (near, far) with weights (p (1 - t), p t); an integral one has weights (p, 0).
//  * Blocks stream through two LDS buffers (block n + 1 is staged while block n is used, one
//    barrier per block); the 16-byte chunks of odd rows are swapped by halves so that the 8 lanes
//    of two adjacent positions hit all 32 banks.
#include "fibattn_device.h"

namespace fibattn {

namespace {

constexpr int kNT = 256;                 // 64 positions x 4 lanes
constexpr int kRowBytes = kD * 2;        // fp16 row
constexpr int kStageRows = 80;           // window block: 64 + W rows, W <= 15
constexpr int kStageRegs = 3;            // 16-byte pieces per thread per staged block
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kXor3 = 0x1B;   // DPP quad_perm: lane ^ 1, ^ 2, ^ 3

__device__ __forceinline__ int swz(int r, int j) { return r * kRowBytes + ((j ^ ((r & 1) << 2)) << 4); }

template <int CTRL> __device__ __forceinline__ uint32_t quad_u(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL> __device__ __forceinline__ float quad_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b), c, false);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    const h2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// 16 dims of LDS row r for lane chunk c: w[0..3] dims 8c..8c+7, w[4..7] dims 32+8c..32+8c+7.
struct Chunk {
    uint32_t w[8];
};

__device__ __forceinline__ Chunk lds_chunk(const char* buf, int r, int c) {
    const uint4 lo = *reinterpret_cast<const uint4*>(buf + swz(r, c));
    const uint4 hi = *reinterpret_cast<const uint4*>(buf + swz(r, c + 4));
    Chunk x;
    x.w[0] = lo.x; x.w[1] = lo.y; x.w[2] = lo.z; x.w[3] = lo.w;
    x.w[4] = hi.x; x.w[5] = hi.y; x.w[6] = hi.z; x.w[7] = hi.w;
    return x;
}

struct Stage {
    uint4 r[kStageRegs];
};

// Rows [j0, j0 + nrows) of one (batch, kv head); rows outside [0, L) are zeros, never loaded.
__device__ __forceinline__ void stage_load(Stage& st, const char* src, int j0, int nrows, int L) {
#pragma unroll
    for (int u = 0; u < kStageRegs; ++u) {
        const int e = threadIdx.x + u * kNT;
        const int row = j0 + (e >> 3);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (e < nrows * 8 && row >= 0 && row < L)
            v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(row) * kRowBytes + (e & 7) * 16);
        st.r[u] = v;
    }
}

__device__ __forceinline__ void stage_store(char* buf, const Stage& st, int nrows) {
#pragma unroll
    for (int u = 0; u < kStageRegs; ++u) {
        const int e = threadIdx.x + u * kNT;
        if (e < nrows * 8) *reinterpret_cast<uint4*>(buf + swz(e >> 3, e & 7)) = st.r[u];
    }
}

// Score of the lane's head c for one key chunk: 4 heads x 8 dot2, DPP reduce-scatter.
__device__ __forceinline__ float quad_score(const uint32_t (&q)[4][8], const Chunk& k) {
    float part[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int m = 0; m < 8; m += 2) {
            a = dot2(q[h][m], k.w[m], a);
            b = dot2(q[h][m + 1], k.w[m + 1], b);
        }
        part[h] = a + b;
    }
    const float s0 = part[0] + quad_f<kXor1>(part[1]);   // head c    from lanes c, c^1
    const float s2 = part[2] + quad_f<kXor1>(part[3]);   // head c^2  from lanes c, c^1
    return s0 + quad_f<kXor2>(s2);                        // head c    from all 4 lanes
}

// o[h][*] += weights . (row r1, row r2) for the 4 heads; wk = this lane's weight pair (fp16 x2).
// The two 8-dim halves of the lane's chunk are read and used one after the other.
__device__ __forceinline__ void pv_pair(float (&o)[4][16], uint32_t wk, const char* buf, int r1, int r2, int c) {
    uint32_t w[4];
    w[0] = wk;
    w[1] = quad_u<kXor1>(wk);
    w[2] = quad_u<kXor2>(wk);
    w[3] = quad_u<kXor3>(wk);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint4 a = *reinterpret_cast<const uint4*>(buf + swz(r1, c + 4 * half));
        const uint4 b = *reinterpret_cast<const uint4*>(buf + swz(r2, c + 4 * half));
        const uint32_t x1[4] = {a.x, a.y, a.z, a.w}, x2[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t lo = __builtin_amdgcn_perm(x2[m], x1[m], 0x05040100u);
            const uint32_t hi = __builtin_amdgcn_perm(x2[m], x1[m], 0x07060302u);
            const int e = 8 * half + 2 * m;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                o[h][e] = dot2(w[h], lo, o[h][e]);
                o[h][e + 1] = dot2(w[h], hi, o[h][e + 1]);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// prep_kv16: rotated keys and values as fp16 rows. Thread = (row, 4 RoPE pairs): 8 threads per
// row, every row of every (batch, head) in parallel.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_kv16_kernel(PrepArgs A) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int quad = static_cast<int>(gid & 7);
    const int64_t row_id = gid >> 3;
    if (row_id >= static_cast<int64_t>(A.n_bh) * A.L) return;
    const int j = static_cast<int>(row_id % A.L);
    const int64_t row = row_id * kD;
    const bf16_t* ks = static_cast<const bf16_t*>(A.k);
    const bf16_t* vs = static_cast<const bf16_t*>(A.v);
    const float4 x1 = load4<bf16_t>(ks + row + 4 * quad);
    const float4 x2 = load4<bf16_t>(ks + row + kPairs + 4 * quad);
    const float4 v1 = load4<bf16_t>(vs + row + 4 * quad);
    const float4 v2 = load4<bf16_t>(vs + row + kPairs + 4 * quad);
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
    store4<f16_t>(A.k16 + row + 4 * quad, make_float4(r1[0], r1[1], r1[2], r1[3]));
    store4<f16_t>(A.k16 + row + kPairs + 4 * quad, make_float4(r2[0], r2[1], r2[2], r2[3]));
    store4<f16_t>(A.v16 + row + 4 * quad, v1);
    store4<f16_t>(A.v16 + row + kPairs + 4 * quad, v2);
}

// ------------------------------------------------------------------------------------------------
// fwd_quad: window W <= MAXW - 1, kept offsets <= MAXK, query heads per key-value head % 4 == 0.
// ------------------------------------------------------------------------------------------------
template <int MAXW, int MAXK>
__global__ __launch_bounds__(kNT, 4) void fwd_quad_kernel(FwdArgs A) {
    constexpr float kNegInf = -__builtin_huge_valf();
    constexpr int NP = MAXW / 2;                       // window weight pairs
    __shared__ __attribute__((aligned(16))) char lds[2][kStageRows * kRowBytes];

    const int p = threadIdx.x >> 2, c = threadIdx.x & 3;
    const int i0 = blockIdx.x * kTile;
    const int n_chunk = A.G >> 2;
    const int g = blockIdx.y / n_chunk;
    const int h0 = g * A.G + (blockIdx.y % n_chunk) * 4;
    const int b = blockIdx.z;
    const int i = i0 + p;
    const int L = A.L, W = A.W;
    const bool active = i < L;

    // kept offsets this tile reaches (a prefix: reach grows with the rung)
    int n_reach = 0;
    for (int n = 0; n < A.n_off; ++n)
        if (i0 + kTile - 1 >= A.off[n].a + A.off[n].interp) n_reach = n + 1;

    const int64_t kv_row0 = (static_cast<int64_t>(b) * A.Hkv + g) * L;
    const char* kbase = static_cast<const char*>(A.kstage) + kv_row0 * kRowBytes;
    const char* vbase = static_cast<const char*>(A.vstage) + kv_row0 * kRowBytes;

    // block sequence: K window, K offsets 0..n_reach-1, V window, V offsets 0..n_reach-1
    const int nblk = 2 * (1 + n_reach);
    auto desc = [&](int blk, const char*& src, int& j0, int& nrows) {
        const int half = 1 + n_reach;
        src = blk < half ? kbase : vbase;
        const int x = blk < half ? blk : blk - half;
        if (x == 0) {
            j0 = i0 - W;
            nrows = kTile + W;
        } else {
            j0 = i0 - A.off[x - 1].a - 1;
            nrows = kTile + 1;
        }
    };
    Stage st;
    int blk = 0, cur = 0;
    {
        const char* src;
        int j0, nr;
        desc(0, src, j0, nr);
        stage_load(st, src, j0, nr, L);
        stage_store(lds[0], st, nr);
        __syncthreads();
    }
    // stage the next block into the other buffer, run `use` on the current one, then one barrier
    // (the other resident workgroups of the CU cover the load latency)
    auto step = [&](auto&& use) {
        if (blk + 1 < nblk) {
            const char* src;
            int j0, nr;
            desc(blk + 1, src, j0, nr);
            stage_load(st, src, j0, nr, L);
            stage_store(lds[cur ^ 1], st, nr);
        }
        use(static_cast<const char*>(lds[cur]));
        __syncthreads();
        cur ^= 1;
        ++blk;
    };

    // ---- q: register slot k holds head h0 + (c ^ k); RoPE'd, times log2(e)/sqrt(D), fp16 ----
    uint32_t q[4][8];
    {
        float2 cs[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) rope_cos_sin(i, A.fr.hi[8 * c + m], A.fr.lo[8 * c + m], cs[m].x, cs[m].y);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
            if (active) {
                const bf16_t* qr = static_cast<const bf16_t*>(A.q) +
                                   ((static_cast<int64_t>(b) * A.Hq + h0 + (c ^ k)) * L + i) * kD;
                lo = *reinterpret_cast<const uint4*>(qr + 8 * c);
                hi = *reinterpret_cast<const uint4*>(qr + kPairs + 8 * c);
            }
            const uint32_t lw[4] = {lo.x, lo.y, lo.z, lo.w}, hw[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float x0 = bf16_lo(lw[m]), x1 = bf16_hi(lw[m]);
                const float y0 = bf16_lo(hw[m]), y1 = bf16_hi(hw[m]);
                const float2 c0 = cs[2 * m], c1 = cs[2 * m + 1];
                q[k][m] = pack_h2((x0 * c0.x - y0 * c0.y) * A.qscale, (x1 * c1.x - y1 * c1.y) * A.qscale);
                q[k][m + 4] = pack_h2((y0 * c0.x + x0 * c0.y) * A.qscale, (y1 * c1.x + x1 * c1.y) * A.qscale);
            }
        }
    }

    // ---- phase A: scores of the lane's head c (base 2) ----
    float s[MAXW + MAXK];
    step([&](const char* buf) {
#pragma unroll
        for (int d = 0; d < MAXW; ++d) {
            s[d] = kNegInf;
            if (d <= W) {
                const float sc = quad_score(q, lds_chunk(buf, p + W - d, c));
                if (active && i >= d) s[d] = sc;
            }
        }
    });
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        s[MAXW + n] = kNegInf;
        if (n < n_reach) {
            step([&](const char* buf) {
                Chunk k = lds_chunk(buf, p + 1, c);
                if (A.off[n].interp) {
                    const Chunk f = lds_chunk(buf, p, c);
                    const _Float16 th = static_cast<_Float16>(A.off[n].t);
                    const h2_t tt = {th, th};
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const h2_t kn = __builtin_bit_cast(h2_t, k.w[m]);
                        const h2_t kf = __builtin_bit_cast(h2_t, f.w[m]);
                        k.w[m] = __builtin_bit_cast(uint32_t, tt * (kf - kn) + kn);
                    }
                }
                const float sc = quad_score(q, k);
                if (active && i >= A.off[n].a + A.off[n].interp) s[MAXW + n] = sc;
            });
        }
    }

    // ---- exact softmax; weights packed in (row, row) pairs as fp16 ----
    float m = kNegInf;
#pragma unroll
    for (int x = 0; x < MAXW + MAXK; ++x) m = fmaxf(m, s[x]);
    if (!active) m = 0.f;
    float l = 0.f;
#pragma unroll
    for (int x = 0; x < MAXW + MAXK; ++x) {
        s[x] = exp2f(s[x] - m);
        l += s[x];
    }
    uint32_t pk[NP + MAXK];
#pragma unroll
    for (int u = 0; u < NP; ++u) pk[u] = pack_h2(s[2 * u], s[2 * u + 1]);
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        const float e = s[MAXW + n];
        const float far = A.off[n].interp ? e * A.off[n].t : 0.f;
        pk[NP + n] = pack_h2(e - far, far);
    }

    // ---- phase B: P.V ----
    float o[4][16];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[h][e] = 0.f;
    step([&](const char* buf) {
#pragma unroll
        for (int u = 0; u < NP; ++u) {
            if (2 * u <= W) {
                const int r1 = p + W - 2 * u;
                const int r2 = (2 * u + 1 <= W) ? r1 - 1 : r1;   // weight 0 when past W
                pv_pair(o, pk[u], buf, r1, r2, c);
            }
        }
    });
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        if (n < n_reach) {
            step([&](const char* buf) {
                pv_pair(o, pk[NP + n], buf, p + 1, p, c);
            });
        }
    }

    // ---- normalise and write ----
    const float inv = 1.0f / l;
    float invk[4];
    invk[0] = inv;
    invk[1] = quad_f<kXor1>(inv);
    invk[2] = quad_f<kXor2>(inv);
    invk[3] = quad_f<kXor3>(inv);
    if (active) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            bf16_t* orow = static_cast<bf16_t*>(A.o) + ((static_cast<int64_t>(b) * A.Hq + h0 + (c ^ k)) * L + i) * kD;
            uint4 lo, hi;
            lo.x = pack_bf16x2(o[k][0] * invk[k], o[k][1] * invk[k]);
            lo.y = pack_bf16x2(o[k][2] * invk[k], o[k][3] * invk[k]);
            lo.z = pack_bf16x2(o[k][4] * invk[k], o[k][5] * invk[k]);
            lo.w = pack_bf16x2(o[k][6] * invk[k], o[k][7] * invk[k]);
            hi.x = pack_bf16x2(o[k][8] * invk[k], o[k][9] * invk[k]);
            hi.y = pack_bf16x2(o[k][10] * invk[k], o[k][11] * invk[k]);
            hi.z = pack_bf16x2(o[k][12] * invk[k], o[k][13] * invk[k]);
            hi.w = pack_bf16x2(o[k][14] * invk[k], o[k][15] * invk[k]);
            *reinterpret_cast<uint4*>(orow + 8 * c) = lo;
            *reinterpret_cast<uint4*>(orow + kPairs + 8 * c) = hi;
        }
        if (A.lse != nullptr)
            A.lse[(static_cast<int64_t>(b) * A.Hq + h0 + c) * L + i] = (m + log2f(l)) * 0.69314718055994530942f;
    }
}

}  // namespace

hipError_t launch_prep_kv16(const PrepArgs& A, hipStream_t s) {
    const int64_t threads = static_cast<int64_t>(A.n_bh) * A.L * 8;
    const unsigned blocks = static_cast<unsigned>((threads + 255) / 256);
    hipLaunchKernelGGL(prep_kv16_kernel, dim3(blocks), dim3(256), 0, s, A);
    return hipGetLastError();
}

bool fwd_quad_supported(const FwdArgs& A) {
    return A.G % 4 == 0 && A.W <= 15 && A.n_off <= 16;
}

hipError_t launch_fwd_quad(const FwdArgs& A, hipStream_t s) {
    dim3 grid((A.L + kTile - 1) / kTile, A.Hkv * (A.G / 4), A.B);
    hipLaunchKernelGGL((fwd_quad_kernel<16, 16>), grid, dim3(kNT), 0, s, A);
    return hipGetLastError();
}

}  // namespace fibattn
