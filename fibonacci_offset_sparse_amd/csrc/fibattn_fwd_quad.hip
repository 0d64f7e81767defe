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
//  * LDS holds statically placed buffers: the window (stored reversed, so the address grows with
//    the distance; keys, then values) and a ring of three offset buffers. Offset blocks are
//    issued two steps ahead, with one barrier per block, and every LDS address is a per-lane
//    base plus an immediate. A sparse L2 warm-up (one 16-byte load per row into a sink slot)
//    runs six blocks ahead, so the real loads hit L2 instead of waiting on HBM. Slots with bit 1 set swap their 64-byte halves, so the 16
//    lanes of 4 adjacent positions spread one ds_read_b128 over all 64 banks.
//  * Staging is LDS DMA (buffer_load ... lds): no VGPRs, issued one block ahead. Rows before 0 or
//    past L fall outside the buffer resource and arrive as zeros, so no row outside [0, L) is
//    ever fetched.
//  * The grid is mapped so that all tiles of one (batch, key-value head) run on one XCD, whose L2
//    then holds that head's keys and values for every tile that re-reads them.
#include "fibattn_device.h"

namespace fibattn {

namespace {

constexpr int kNT = 256;                 // 64 positions x 4 lanes
constexpr int kRowBytes = kD * 2;        // one fp16 row
// LDS: separate arrays (so the compiler can tell a DMA into one from reads of another) of 128-byte
// slots: the window (64 + W <= 79 rows, reversed; keys, then values), a ring of three offset
// buffers (65 rows used, 72 = 9 DMA groups allocated), and a 1 KB sink for surplus and warm-up
// loads. Every wave issues a fixed number of DMA instructions per step, so the waits can count.
constexpr int kWinSlots = 80;
constexpr int kRingSlots = 72;
constexpr int kRing = 3;
constexpr int kWarmAhead = 6;                              // L2 warm-up distance, in blocks
constexpr int kXor1 = 0xB1, kXor2 = 0x4E, kXor3 = 0x1B;   // DPP quad_perm: lane ^ 1, ^ 2, ^ 3
constexpr int kRsrcWord3 = 0x00020000;                    // raw buffer, gfx9 family
#ifndef FIBATTN_FWD_WGS_PER_CU
#define FIBATTN_FWD_WGS_PER_CU 3
#endif
// Workgroups per CU the register budget is sized for: 3 gives 168 VGPRs, enough to hold the
// 64 output accumulators and 24 weight pairs of the P.V phase without spilling (a spill reload
// is a vector-memory load and would wait behind every staging load in flight).
constexpr int kWgsPerCu = FIBATTN_FWD_WGS_PER_CU;

// Byte address of 16-byte chunk j of LDS slot s. Slots with bit 1 set swap their two 64-byte
// halves: a ds_read_b128 serves 16 lanes (4 positions, 4 consecutive rows) at a time over 64 banks
// (256 bytes), and rows r..r+3 then put their 64 bytes into 4 different quarters of the banks.
__device__ __forceinline__ int chunk_addr(int s, int j) { return s * kRowBytes + ((j ^ (((s >> 1) & 1) << 2)) << 4); }

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

// Wait until at most N vector-memory instructions of this wave are in flight (its LDS DMAs up to
// the block the next step reads have landed), then the workgroup barrier. __syncthreads would
// also drain every in-flight prefetch.
template <int N> __device__ __forceinline__ void publish() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint4 lds16(const char* lds, int addr) {
    return *reinterpret_cast<const uint4*>(lds + addr);
}

// 16 dims of one row for lane chunk c: w[0..3] dims 8c..8c+7, w[4..7] dims 32+8c..32+8c+7.
struct Chunk {
    uint32_t w[8];
};

__device__ __forceinline__ Chunk lds_chunk(const char* lds, int lo_addr, int hi_addr) {
    const uint4 lo = lds16(lds, lo_addr), hi = lds16(lds, hi_addr);
    Chunk x;
    x.w[0] = lo.x; x.w[1] = lo.y; x.w[2] = lo.z; x.w[3] = lo.w;
    x.w[4] = hi.x; x.w[5] = hi.y; x.w[6] = hi.z; x.w[7] = hi.w;
    return x;
}

// Score of the lane's head c for one key chunk: 4 heads x 8 dot2, DPP reduce-scatter.
__device__ __forceinline__ float quad_score(const uint32_t (&q)[4][8], const Chunk& k) {
    float part[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        float a = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) a = dot2(q[h][m], k.w[m], a);
        part[h] = a;
    }
    const float s0 = part[0] + quad_f<kXor1>(part[1]);   // head c    from lanes c, c^1
    const float s2 = part[2] + quad_f<kXor1>(part[3]);   // head c^2  from lanes c, c^1
    return s0 + quad_f<kXor2>(s2);                        // head c    from all 4 lanes
}

// o[h][*] += (w1, w2) . (row 1, row 2) for the 4 heads; wk = this lane's weight pair (fp16 x2),
// the other heads' pairs come from the quad. The two 8-dim halves are used one after the other.
__device__ __forceinline__ void pv_pair(float (&o)[4][16], uint32_t wk, const char* lds, int r1_lo, int r1_hi,
                                        int r2_lo, int r2_hi) {
    uint32_t w[4];
    w[0] = wk;
    w[1] = quad_u<kXor1>(wk);
    w[2] = quad_u<kXor2>(wk);
    w[3] = quad_u<kXor3>(wk);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint4 a = lds16(lds, half ? r1_hi : r1_lo);
        const uint4 b = lds16(lds, half ? r2_hi : r2_lo);
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
// prep_kv16: rotated keys and values as fp16 rows, plus the cos/sin table of every position (for
// the queries). Thread = (row, 4 RoPE pairs): 8 threads per row, every row in parallel.
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
    float2 cs[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        rope_cos_sin(j, A.fr.hi[4 * quad + u], A.fr.lo[4 * quad + u], cs[u].x, cs[u].y);
        r1[u] = a[u] * cs[u].x - b[u] * cs[u].y;
        r2[u] = b[u] * cs[u].x + a[u] * cs[u].y;
    }
    store4<f16_t>(A.k16 + row + 4 * quad, make_float4(r1[0], r1[1], r1[2], r1[3]));
    store4<f16_t>(A.k16 + row + kPairs + 4 * quad, make_float4(r2[0], r2[1], r2[2], r2[3]));
    store4<f16_t>(A.v16 + row + 4 * quad, v1);
    store4<f16_t>(A.v16 + row + kPairs + 4 * quad, v2);
    if (row_id < A.L) {   // the first (batch, head) writes the table: [L][32] (cos, sin)
        float4* t = reinterpret_cast<float4*>(A.cs + (static_cast<int64_t>(j) * kPairs + 4 * quad) * 2);
        t[0] = make_float4(cs[0].x, cs[0].y, cs[1].x, cs[1].y);
        t[1] = make_float4(cs[2].x, cs[2].y, cs[3].x, cs[3].y);
    }
}

// ------------------------------------------------------------------------------------------------
// fwd_quad: window W <= MAXW - 1, kept offsets <= MAXK, query heads per key-value head % 4 == 0.
// ------------------------------------------------------------------------------------------------
template <int MAXW, int MAXK>
__global__ __launch_bounds__(kNT, kWgsPerCu) void fwd_quad_kernel(FwdArgs A) {
    constexpr float kNegInf = -__builtin_huge_valf();
    constexpr int NP = MAXW / 2;                       // window weight pairs
    __shared__ __attribute__((aligned(1024))) char ldsW[kWinSlots * kRowBytes];
    __shared__ __attribute__((aligned(1024))) char ldsR0[kRingSlots * kRowBytes];
    __shared__ __attribute__((aligned(1024))) char ldsR1[kRingSlots * kRowBytes];
    __shared__ __attribute__((aligned(1024))) char ldsR2[kRingSlots * kRowBytes];
    __shared__ __attribute__((aligned(1024))) char ldsSink[1024];

    const int p = threadIdx.x >> 2, c = threadIdx.x & 3;
    const int L = A.L, W = A.W;
    const int n_tiles = (L + kTile - 1) / kTile;
    const int n_chunk = A.G >> 2;
    // workgroup -> (unit, tile); with the XCD map, unit u runs on XCD u % 8 for all its tiles
    int unit, tile;
    {
        const int w = blockIdx.x;
        if (A.xcd_map) {
            const int sl = w >> 3;
            unit = (sl / n_tiles) * 8 + (w & 7);
            tile = sl % n_tiles;
        } else {
            unit = w / n_tiles;
            tile = w % n_tiles;
        }
    }
    const int chunk = unit % n_chunk;
    const int bg = unit / n_chunk;                      // b * Hkv + g
    const int b = bg / A.Hkv;
    const int h0 = (bg % A.Hkv) * A.G + chunk * 4;
    const int i0 = tile * kTile;
    const int i = i0 + p;
    const bool active = i < L;

    // kept offsets this tile reaches (a prefix: the reach grows with the rung)
    int n_reach = 0;
    for (int n = 0; n < A.n_off; ++n)
        if (i0 + kTile - 1 >= A.off[n].a + A.off[n].interp) n_reach = n + 1;

    // ---- per-lane LDS addresses (everything else is an immediate) ----
    const int s0 = kWinSlots - 1 - p - W;               // window slot of distance 0
    int wl[4];                                          // window chunk c for distances d = e mod 4
#pragma unroll
    for (int e = 0; e < 4; ++e) wl[e] = chunk_addr(s0 + e, c) - e * kRowBytes;
    auto whi = [](int lo) { return lo ^ 64; };          // chunk c + 4: the other half of the slot
    const int nl = chunk_addr(p + 1, c), nh = chunk_addr(p + 1, c + 4);   // offset block: near row
    const int fl = chunk_addr(p, c), fh = chunk_addr(p, c + 4);           // far row

    // ---- staging: LDS DMA (buffer_load ... lds) of one (batch, kv head). Rows outside [0, L) fall
    // outside the buffer and arrive as zeros. A wave instruction fills 1 KB = 8 slots: lane l
    // lands on slot 8g + (l >> 3), physical chunk l & 7, so it fetches that slot's row and the
    // logical chunk the swizzle puts there. Wave w issues groups g = w, w + 4, w + 8: always 3
    // instructions, groups past the block going to the sink.
    const int64_t kv_row0 = static_cast<int64_t>(bg) * L;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(A.kstage) + kv_row0 * kRowBytes), 0, L * kRowBytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(static_cast<const char*>(A.vstage) + kv_row0 * kRowBytes), 0, L * kRowBytes, kRsrcWord3);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lrow = lane >> 3;
    const int lchunk = ((lane & 7) ^ (((lrow >> 1) & 1) << 2)) << 4;
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    auto dma = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int row) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, row * kRowBytes + lchunk, 0, 0, 0);
    };
    // window block: rows j0 + r, r < 64 + W, at slot 79 - r (10 groups)
    auto stage_window = [&](const __amdgpu_buffer_rsrc_t& rs) {
        const int j0 = i0 - W;
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int g = wave + 4 * u;
            const int r = kWinSlots - 1 - (8 * g + lrow);
            dma(rs, g < kWinSlots / 8 ? ldsW + g * 1024 : ldsSink, j0 + r);
        }
    };
    // offset block n (or only sink loads when n >= n_reach): rows j0 + r at slot r (9 groups)
    auto stage_offset = [&](const __amdgpu_buffer_rsrc_t& rs, char* ring_buf, int n) {
        const bool real = n < n_reach;
        const int j0 = real ? i0 - A.off[n].a - 1 : -(kRingSlots + 1);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int g = wave + 4 * u;
            dma(rs, (real && g < kRingSlots / 8) ? ring_buf + g * 1024 : ldsSink, j0 + 8 * g + lrow);
        }
    };
    // L2 warm-up of block x of [key offsets, value window, value offsets]: wave w touches 16 rows,
    // one line each, into the sink (one instruction per wave; a dummy out-of-range load past the end)
    auto warm = [&](int x) {
        const bool real = x < 2 * n_reach + 1;
        int j0 = -(kTile + kWinSlots);
        if (real) j0 = (x == n_reach) ? i0 - W : i0 - A.off[x < n_reach ? x : x - n_reach - 1].a - 1;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(x < n_reach ? krs : vrs, (lds_ptr_t)ldsSink, 16,
                                                 (j0 + 16 * wave + (lane >> 2)) * kRowBytes + ((lane & 3) << 4),
                                                 0, 0, 0);
    };
    auto ring = [&](int k) -> char* { return k == 0 ? ldsR0 : (k == 1 ? ldsR1 : ldsR2); };

    stage_window(krs);                                  // key window (3 instructions, before q)

    // ---- q: register slot k holds head h0 + (c ^ k); RoPE'd, times log2(e)/sqrt(D), fp16 ----
    uint32_t q[4][8];
    {
        float2 cs[8];
        const float4* ct = reinterpret_cast<const float4*>(A.cstab) +
                           (static_cast<int64_t>(active ? i : 0) * kPairs + 8 * c) / 2;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 t = ct[m];
            cs[2 * m] = make_float2(t.x, t.y);
            cs[2 * m + 1] = make_float2(t.z, t.w);
        }
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
    stage_offset(krs, ldsR0, 0);
    stage_offset(krs, ldsR1, 1);
#pragma unroll
    for (int x = 2; x < 2 + kWarmAhead; ++x) warm(x);
    publish<12>();                                      // the key window has landed

    // ---- phase A: scores of the lane's head c (base 2) ----
    // Ring schedule: key offset block j sits in ring j % 3. The window step issues block 2; step j
    // issues block j + 2 (the value window at step 0) into the ring step j - 1 released. Each step
    // issues 4 instructions per wave (a 3-instruction block, one warm-up); the wait before each
    // barrier lets exactly the loads issued after the next step's block stay in flight.
    float s[MAXW + MAXK];
    stage_offset(krs, ldsR2, 2);
    warm(2 + kWarmAhead);
#pragma unroll
    for (int d = 0; d < MAXW; ++d) {
        s[d] = kNegInf;
        if (d <= W) {
            const int a = wl[d & 3] + d * kRowBytes;
            const float sc = quad_score(q, lds_chunk(ldsW, a, whi(a)));
            s[d] = (active && i >= d) ? sc : kNegInf;
        }
    }
    if (n_reach == 0) {                                 // no offsets: bring in the value window now
        publish<0>();
        stage_window(vrs);
        publish<0>();
    } else {
        publish<13>();                                  // block 0 (13 loads issued after it) landed
    }
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        s[MAXW + n] = kNegInf;
        if (n < n_reach) {
            if (n == 0)
                stage_window(vrs);
            else
                stage_offset(krs, ring((n + 2) % kRing), n + 2);
            warm(n + 3 + kWarmAhead);
            const char* buf = ring(n % kRing);
            Chunk k = lds_chunk(buf, nl, nh);
            if (A.off[n].interp) {
                const Chunk f = lds_chunk(buf, fl, fh);
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
            s[MAXW + n] = (active && i >= A.off[n].a + A.off[n].interp) ? sc : kNegInf;
            if (n + 1 == n_reach)
                publish<0>();                           // next: the value window, issued at step 0
            else if (n == 0)
                publish<14>();
            else if (n == 1)
                publish<9>();
            else
                publish<5>();
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
    // value offset block j sits in ring j % 3; the window step issues blocks 0, 1, 2 (every ring is
    // free after the last key step), step j >= 1 issues block j + 2
    float o[4][16];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[h][e] = 0.f;
    stage_offset(vrs, ldsR0, 0);
    stage_offset(vrs, ldsR1, 1);
    stage_offset(vrs, ldsR2, 2);
    warm(n_reach + 1 + kWarmAhead);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        if (2 * u <= W) {
            // slots 2u and 2u + 1 are adjacent rows; past W the second weight is 0 (reread row 1)
            const int a1 = wl[(2 * u) & 3] + 2 * u * kRowBytes;
            const int a2 = (2 * u + 1 <= W) ? wl[(2 * u + 1) & 3] + (2 * u + 1) * kRowBytes : a1;
            pv_pair(o, pk[u], ldsW, a1, whi(a1), a2, whi(a2));
        }
    }
    if (n_reach > 0) publish<7>();                      // value block 0 has landed
#pragma unroll
    for (int n = 0; n < MAXK; ++n) {
        if (n < n_reach) {
            if (n >= 1) stage_offset(vrs, ring((n + 2) % kRing), n + 2);
            warm(n_reach + 2 + n + kWarmAhead);
            pv_pair(o, pk[NP + n], ring(n % kRing), nl, nh, fl, fh);
            if (n + 1 == n_reach) {
                // last block: nothing left to publish
            } else if (n == 0) {
                publish<5>();
            } else if (n == 1) {
                publish<6>();
            } else {
                publish<5>();
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no DMA may outlive the workgroup

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

hipError_t launch_fwd_quad(const FwdArgs& A0, hipStream_t s) {
    FwdArgs A = A0;
    const int64_t n_tiles = (A.L + kTile - 1) / kTile;
    const int64_t n_units = static_cast<int64_t>(A.B) * A.Hkv * (A.G / 4);
    A.xcd_map = (n_units % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((fwd_quad_kernel<16, 16>), dim3(static_cast<unsigned>(n_units * n_tiles)), dim3(kNT), 0, s,
                       A);
    return hipGetLastError();
}

}  // namespace fibattn
