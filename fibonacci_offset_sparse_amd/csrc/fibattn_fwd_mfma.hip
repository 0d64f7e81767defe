// Forward attention for bfloat16 storage on gfx950: the fast kernel, on the matrix cores.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv
// 2606.28560), §2 "Attended set": window distances 0..W plus one slot per rung at distance
// d = alpha f, read by linear interpolation between rows i - floor(d) and i - floor(d) - 1, with
// RoPE applied before the gather. Offsets are shared by all queries, so for a tile of 64 queries
// each slot reads one contiguous block of rows.
//
// Inputs come from prep_kv16: keys rotated at their positions and values, both as fp16 rows of
// 128 bytes with dims permuted (element 4m + c holds dim 16c + m), and the cos/sin table. A
// workgroup owns (batch b, key-value head g, 4 query heads, 64 positions); wave w takes positions
// 16w..16w+15 of the tile.
//
// Every position is its own small product: its 4 query heads (they share the key-value head)
// against the rows its slots read. v_mfma_f32_4x4x4_16b_f16 computes 16 independent 4x4x4
// blocks, one per position of the wave; lane 4p' + x is row x of the A operand and column x of
// the B operand and of the result, of block p'.
//
//  * Virtual slots: a window distance is one row; an interpolated rung is two rows, near (the
//    nearer row, coefficient 1 - t) and far (coefficient t). Scores and outputs are linear in
//    the blended row, so q.(blend) = (1 - t) q.near + t q.far, and the value blend spreads its
//    weight p as p (1 - t), p t. An integral rung keeps t = 0. Groups of 4 virtual slots are
//    4 window distances, or (near, far) of two consecutive rungs.
//  * QK: A = the 4 rows of the group (lane x reads virtual slot x's row), B = q of head x in the
//    keys' permuted order, K = 64 dims in 16 products. The result lane (p', x) holds head x's 4
//    scores: all of a lane's scores stay in its registers, the softmax is exact and in-lane
//    (base 2).
//  * PV: A = head x's 4 weights (the same lane), B = the 4 rows' element 4m + x, read with the
//    transposing ds_read_b64_tr_b16 from the permuted values (dim 16x + m), 16 products cover 64
//    dims; the result lane (p', x) holds dims 16x..16x+15 of all 4 heads.
//  * LDS: two staging buffers of 18 KB (four workgroups per CU), used in turn by a sequence of
//    items: the key near block (rows i0 - 64 .. i0 + 63: the window and both rows of every rung
//    with floor(d) <= 63), the key far steps (two larger rungs of 65 rows each), the value near
//    block, the value far steps. Staging is LDS DMA (buffer_load ... lds): no VGPRs; rows before
//    0 or past L fall outside the buffer resource and arrive as zeros, so every row a lane reads
//    is finite. Each item is issued while the one before it is being computed on, with one
//    barrier per item after a counted vmcnt wait.
//  * Banks: 16-byte chunk k of slot s sits at chunk k ^ ((s >> 1) & 7), so the same chunk of 16
//    consecutive slots covers all 64 banks, and the second rung's block sits two slots up. Key
//    reads (16 lanes per pass) are then free of bank conflicts for window groups and far steps,
//    and for a near rung pair whose floors differ by d with d mod 32 in 0..11 or 21..27 (2-way
//    otherwise); the transposing value reads are free for window groups and 2-way for rung
//    groups (a 32-lane pass reads 18 distinct rows).
//  * The grid is mapped so that all tiles of one (batch, key-value head) run on one XCD, whose L2
//    then holds that head's keys and values for every tile that re-reads them, and each CU mixes
//    early and late tiles.
//  * q arrives by non-temporal LDS DMA (read once) and o and lse leave by non-temporal stores.
#include "fibattn.h"
#include "fibattn_mfma.h"

namespace fibattn {

namespace {

using namespace mx;

// Workgroups per CU: LDS is 2 x 18 KB per workgroup, so four fit (1024 workgroups at the paper's
// shape are one wave of the grid); the register budget this gives (128 per lane) must hold q,
// the scores and the 64 output accumulators without spilling (a spill reload is a vector-memory
// load and would wait behind every staging load in flight).
constexpr int kWgsPerCu = 4;

// ---- phase trace (in the build with FIBATTN_PHASE_TRACE only) ----
// Per workgroup of the attention kernel (wave 0), six stamps of the 100 MHz real-time counter:
// start, key near block landed, key pass done, value near block landed, value pass done, outputs
// stored (after a wait for the stores); then the tile and its counts of kept rungs and steps, and the
// CU. In the usual build every PhaseClock call is empty.
#ifdef FIBATTN_PHASE_TRACE
constexpr int kTraceWgs = 65536;
constexpr int kTraceWords = 8;
__device__ uint64_t g_phase[kTraceWgs * kTraceWords];
struct PhaseClock {
    uint64_t t[6];
    __device__ __forceinline__ void mark(int k) { t[k] = __builtin_amdgcn_s_memrealtime(); }
    __device__ __forceinline__ void record(int tile, int n_steps, int kn, int n_reach) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        mark(5);
        if (threadIdx.x == 0 && blockIdx.x < static_cast<unsigned>(kTraceWgs)) {
            uint64_t* g = g_phase + static_cast<uint64_t>(blockIdx.x) * kTraceWords;
#pragma unroll
            for (int k = 0; k < 6; ++k) g[k] = t[k];
            g[6] = static_cast<uint64_t>(tile) | (static_cast<uint64_t>(n_steps) << 16) |
                   (static_cast<uint64_t>(kn) << 24) | (static_cast<uint64_t>(n_reach) << 32);
            g[7] = static_cast<uint64_t>(__smid());
        }
    }
};
#else
struct PhaseClock {
    __device__ __forceinline__ void mark(int) {}
    __device__ __forceinline__ void record(int, int, int, int) {}
};
#endif

// ------------------------------------------------------------------------------------------------
// prep_kv16: rotated keys and values as fp16 rows, plus the cos/sin table of every position. One
// layout, read by the forward and the backward alike: both keys and values have their dims
// permuted, element 4m + c holding dim 16c + m, so that a transposing LDS read of 4 consecutive
// elements gives a lane 4 rows of its own 16 dims (a contraction over dims, as in the scores, reads
// the permuted rows against a query permuted the same way). Thread u of a row writes elements
// 8u..8u+7: dims 16e + 2u (e < 4) and 16(e - 4) + 2u + 1, which hold RoPE pairs 2u, 2u + 1,
// 16 + 2u, 17 + 2u whole (pair m: dims m and m + 32). The table is cos and sin as they are.
// ------------------------------------------------------------------------------------------------
// A thread takes one position j and kPrepRows (batch, head) rows of it: every row's loads are
// issued first, then the cos/sin of its 4 RoPE pairs are computed once for all of them. Workgroup
// (x, y) = (positions 32x .. 32x + 31, row group y: kPrepRows consecutive (batch, head) rows).
//
// Range flags. fp16 holds a rotated key or value row exactly enough only inside a range: every
// element below 2^15 in magnitude (65504 is fp16's largest) and, unless the row is zero, a row
// maximum of at least 2^-10 (below that the row's largest elements come near fp16's subnormals,
// 2^-14, where relative precision is lost). Each wave writes one byte of its workgroup's word (its
// 8 positions of the block), nonzero when a key or value row there lies outside; the attention
// kernels check the words of the rows they read and compute such tiles in float32 from the
// caller's bf16 rows instead. A row's 8 threads find its largest magnitude over 8 lanes (DPP).
constexpr int kPrepRows = kPrepRowGroup;

// MAIN: the staged rows, the table and the flags; LO: the low parts of the rotated keys.
template <bool MAIN, bool LO>
__global__ __launch_bounds__(256) void prep_kv16_kernel(PrepArgs A) {
    const int u = threadIdx.x & 7;
    const int grp = blockIdx.y;
    const int j = 32 * blockIdx.x + (threadIdx.x >> 3);
    const bool active = j < A.L;
    const int jc = active ? j : 0;                      // rows past L are never read
    const bf16_t* ks = static_cast<const bf16_t*>(A.k);
    const bf16_t* vs = static_cast<const bf16_t*>(A.v);
    // the thread's pairs 2u, 2u + 1, 16 + 2u, 17 + 2u, and their frequencies (loaded ahead of the
    // rows: a wait for them then does not wait for the rows too)
    int pr[4];
    float fh[4], fl[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pr[e] = (e >> 1) * 16 + 2 * u + (e & 1);
        fh[e] = A.fr.hi[pr[e]];
        fl[e] = A.fr.lo[pr[e]];
    }
    // loads of every row (dims 16c + 2u, 16c + 2u + 1, c = 0..3, of the key and the value), in
    // flight while the cos/sin are computed
    uint32_t kw[kPrepRows][4], vw[kPrepRows][4];
#pragma unroll
    for (int r = 0; r < kPrepRows; ++r) {
        const int bh = grp * kPrepRows + r;
        const int64_t row = (static_cast<int64_t>(bh < A.n_bh ? bh : 0) * A.L + jc) * kD;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            kw[r][c] = *reinterpret_cast<const uint32_t*>(ks + row + 16 * c + 2 * u);
            vw[r][c] = MAIN ? *reinterpret_cast<const uint32_t*>(vs + row + 16 * c + 2 * u) : 0u;
        }
    }
    // the cos/sin: computed by the main pass, read back from its table by a pass that writes only
    // the low parts (so both rotate the key with the very same values)
    float2 cs[4];
    if constexpr (MAIN) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rope_cos_sin(jc, fh[e], fl[e], cs[e].x, cs[e].y);
    } else {
        const float2* t = reinterpret_cast<const float2*>(A.cs) + static_cast<int64_t>(jc) * kPairs;
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[e] = t[pr[e]];
    }
    if (MAIN && grp == 0 && active) {   // the table: [L][32] (cos, sin)
        float2* t = reinterpret_cast<float2*>(A.cs) + static_cast<int64_t>(j) * kPairs;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[pr[e]] = cs[e];
    }
    bool outside = false;                               // a row of the thread's group lies outside
    float elem_max = 0.f;                               // the thread's largest element of every row
#pragma unroll
    for (int r = 0; r < kPrepRows; ++r) {
        const int bh = grp * kPrepRows + r;
        const bool live = active && bh < A.n_bh;        // uniform over the 8 threads of a row
        const int64_t row = (static_cast<int64_t>(live ? bh : 0) * A.L + jc) * kD;
        // x, y of pairs 2u, 2u + 1 (dims 2u, 2u + 1 and 32 + ..) and 16 + 2u, 17 + 2u
        const float x[4] = {bf16_lo(kw[r][0]), bf16_hi(kw[r][0]), bf16_lo(kw[r][1]), bf16_hi(kw[r][1])};
        const float y[4] = {bf16_lo(kw[r][2]), bf16_hi(kw[r][2]), bf16_lo(kw[r][3]), bf16_hi(kw[r][3])};
        float rx[4], ry[4];
        float kmax = 0.f, vmax = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // the rotated key rounded to float32 first, in every instantiation alike (the staged
            // fp16 row and its low part may come from different passes): explicit fused forms, and
            // an empty asm that keeps the compiler from folding the fp16 conversion into the fma
            // (which would round the exact value once instead)
            rx[e] = fmaf(x[e], cs[e].x, -(y[e] * cs[e].y));
            ry[e] = fmaf(y[e], cs[e].x, x[e] * cs[e].y);
            asm volatile("" : "+v"(rx[e]), "+v"(ry[e]));
            kmax = fmaxf(kmax, fmaxf(fabsf(rx[e]), fabsf(ry[e])));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) vmax = fmaxf(vmax, fmaxf(fabsf(bf16_lo(vw[r][c])), fabsf(bf16_hi(vw[r][c]))));
        if constexpr (MAIN) {
            const float km = oct_max(live ? kmax : 0.f), vm = oct_max(live ? vmax : 0.f);
            outside |= (km > 0.f && km < kFp16Small) || (vm > 0.f && vm < kFp16Small);
            elem_max = fmaxf(elem_max, live ? fmaxf(kmax, vmax) : 0.f);
        }
        if (!live) continue;
        // element 8u + e: e < 4 is dim 16e + 2u, e >= 4 is dim 16(e - 4) + 2u + 1
        if constexpr (MAIN) {
            store4<f16_t>(A.k16 + row + 8 * u, make_float4(rx[0], rx[2], ry[0], ry[2]));
            store4<f16_t>(A.k16 + row + 8 * u + 4, make_float4(rx[1], rx[3], ry[1], ry[3]));
            store4<f16_t>(A.v16 + row + 8 * u,
                          make_float4(bf16_lo(vw[r][0]), bf16_lo(vw[r][1]), bf16_lo(vw[r][2]), bf16_lo(vw[r][3])));
            store4<f16_t>(A.v16 + row + 8 * u + 4,
                          make_float4(bf16_hi(vw[r][0]), bf16_hi(vw[r][1]), bf16_hi(vw[r][2]), bf16_hi(vw[r][3])));
        }
        if constexpr (LO) {
            // what fp16 rounding left out of each rotated key element: a second fp16 operand
            // whose product with q restores the score to about 2^-22 relative
            auto lo = [](float v) { return v - static_cast<float>(static_cast<_Float16>(v)); };
            store4<f16_t>(A.k16lo + row + 8 * u, make_float4(lo(rx[0]), lo(rx[2]), lo(ry[0]), lo(ry[2])));
            store4<f16_t>(A.k16lo + row + 8 * u + 4, make_float4(lo(rx[1]), lo(rx[3]), lo(ry[1]), lo(ry[3])));
        }
    }
    if constexpr (MAIN) {
        const bool any = __builtin_amdgcn_ballot_w64(outside || elem_max >= kFp16Big) != 0;
        if ((threadIdx.x & 63) == 0)
            reinterpret_cast<uint8_t*>(A.flags)[(static_cast<int64_t>(grp) * A.n_blk + blockIdx.x) * 4 + (threadIdx.x >> 6)] =
                any ? 1 : 0;
    }
}

// ------------------------------------------------------------------------------------------------
// The float32 tile: a tile computed from the caller's bf16 rows (q, k, v) and the cos/sin table,
// for tiles whose rows lie outside the range the fp16 staging holds (the prep's range flags, or q
// itself). Thread 8p' + e takes dims 8e .. 8e + 7 of position i0 + p' (an 8-lane group holds a whole
// row; sums over dims close with three DPP steps), 32 positions at a time, one query head after
// another, with an online softmax over the slots in the order window, rungs. Rows come straight from
// global memory: slow, and only for such tiles. It runs inside the matrix-core kernels, so it is
// written to need few registers.
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ void fwd_tile_fp32(const FwdArgs& A, int b, int bg, int h0, int i0) {
    constexpr float kNegInf = -__builtin_huge_valf();
    const int e = threadIdx.x & 7, L = A.L;
    const bf16_t* kb = static_cast<const bf16_t*>(A.k) + static_cast<int64_t>(bg) * L * kD;
    const bf16_t* vb = static_cast<const bf16_t*>(A.v) + static_cast<int64_t>(bg) * L * kD;
    const int n_slots = A.W + 1 + A.n_off;
#pragma unroll 1
    for (int it = 0; it < 2 * 4; ++it) {                // (half of the tile, head)
        const int i = i0 + 32 * (it & 1) + (threadIdx.x >> 3);
        if (i >= L) continue;                           // whole 8-lane groups skip together
        const int64_t qrow = (static_cast<int64_t>(b) * A.Hq + h0 + (it >> 1)) * L + i;
        float qv[8], o[8], row[8];
        rot_eighth(static_cast<const bf16_t*>(A.q) + qrow * kD, A.cstab, i, e, qv);
        float m = kNegInf, l = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            qv[u] *= A.qscale;                          // scores in base 2
            o[u] = 0.f;
        }
#pragma unroll 1
        for (int sl = 0; sl < n_slots; ++sl) {
            // slot sl: window distance sl, or kept rung sl - W - 1: rows j (weight 1 - t), j - 1 (t)
            int j;
            float t = 0.f;
            if (sl <= A.W) {
                j = i - sl;
            } else {
                const int n = sl - A.W - 1;
                j = i - A.off[n].a;
                if (A.off[n].interp) {
                    t = A.off[n].t;
                    --j;                                 // the far row must exist too
                }
                if (j < 0) continue;
                j += A.off[n].interp;
            }
            if (j < 0) continue;
            // the score and the value are linear in the blended row: each row once
            float sc = 0.f;
#pragma unroll 1
            for (int r = 0; r < (t != 0.f ? 2 : 1); ++r) {
                rot_eighth(kb + static_cast<int64_t>(j - r) * kD, A.cstab, j - r, e, row);
                float d = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) d = fmaf(qv[u], row[u], d);
                sc += (r ? t : 1.f - t) * oct_sum(d);
            }
            const float mn = fmaxf(m, sc);
            const float keep = __builtin_amdgcn_exp2f(m - mn), w = __builtin_amdgcn_exp2f(sc - mn);
            l = fmaf(l, keep, w);
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] *= keep;
#pragma unroll 1
            for (int r = 0; r < (t != 0.f ? 2 : 1); ++r) {
                const uint4 vw = reinterpret_cast<const uint4*>(vb + static_cast<int64_t>(j - r) * kD)[e];
                const uint32_t v4[4] = {vw.x, vw.y, vw.z, vw.w};
                const float wr = w * (r ? t : 1.f - t);
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    o[2 * h] = fmaf(wr, bf16_lo(v4[h]), o[2 * h]);
                    o[2 * h + 1] = fmaf(wr, bf16_hi(v4[h]), o[2 * h + 1]);
                }
            }
            m = mn;
        }
        const float inv = 1.0f / l;
        const uint4 ov = make_uint4(pack_bf2(o[0] * inv, o[1] * inv), pack_bf2(o[2] * inv, o[3] * inv),
                                    pack_bf2(o[4] * inv, o[5] * inv), pack_bf2(o[6] * inv, o[7] * inv));
        store_nt(static_cast<bf16_t*>(A.o) + qrow * kD + 8 * e, ov);
        if (e == 0 && A.lse != nullptr) store_nt(A.lse + qrow, (m + log2f(l)) * 0.69314718055994530942f);
    }
}

// Whether a query row (64 bf16 values in r) scaled by qscale lies outside what fp16 holds exactly
// enough once rotated (rotation moves each element by at most a factor sqrt(2) either way).
__device__ __forceinline__ bool q_outside_fp16(const uint4 (&r)[8], float qscale) {
    const float mx = bf16_bits_value(max_abs_bf16_bits(r)) * qscale;
    return mx >= 0.5f * kFp16Big || (mx > 0.f && mx < 2.f * kFp16Small);
}

// ------------------------------------------------------------------------------------------------
// fwd_mfma: W <= 15 (4 window groups), kept rungs <= 2 MAXS, query heads per key-value head % 4 == 0.
// INT: every kept rung is integral (the integer-offset path of §2 "Implementation note"): a rung
// reads one row, so the rungs with a <= 64 are read from the near block four to a group (at most
// two groups), and a far step stages its two rungs as 64-row blocks, with no blending of rows.
// ------------------------------------------------------------------------------------------------
template <int MAXS, bool INT>
__global__ __launch_bounds__(kNT, kWgsPerCu) void fwd_mfma_kernel(FwdArgs A) {
    constexpr float kNegInf = -__builtin_huge_valf();
    constexpr int MAXK = 2 * MAXS;
    // Two staging buffers used in turn. An item is the key near block (the window and the rungs
    // with a <= 63), a far step of two key rungs, the value near block or a far step of two value
    // rungs. The near block holds rows i0 - 64 + s at slot s; a far step holds rung 2k at slot 0
    // (block A) and rung 2k + 1 at slot kBlkSlots (block B). Two arrays, always named at compile
    // time where they are read: the compiler then knows an LDS read does not touch the buffer the
    // DMA in flight fills.
    __shared__ __attribute__((aligned(1024))) char lds0[kBufBytes];
    __shared__ __attribute__((aligned(1024))) char lds1[kBufBytes];
    __shared__ int votes[4];                            // per wave: a row of the tile lies outside fp16's range

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int pq = lane >> 2, x = lane & 3;             // position within the wave, quad lane
    const int p = 16 * wave + pq;                       // position within the tile
    const int L = A.L, W = A.W;
    const int n_tiles = (L + kTile - 1) / kTile;
    const int n_chunk = A.G >> 2;
    int unit, tile;
    unit_tile(blockIdx.x, n_tiles, A.xcd_map, unit, tile);
    const int chunk = unit % n_chunk;
    const int bg = unit / n_chunk;                      // b * Hkv + g
    const int b = bg / A.Hkv;
    const int h0 = (bg % A.Hkv) * A.G + chunk * 4;
    const int i0 = tile * kTile;
    const int i = i0 + p;
    const bool active = i < L;
    PhaseClock clk;
    clk.mark(0);

    // kept rungs this tile reaches (a prefix: the reach grows with the rung), in steps of two
    // (counted over the packed scan table, RungScan: a few wide scalar loads, where a loop over
    // the offset table waits for each rung's load in turn)
    int n_reach = 0, n_lo = 0;
#pragma unroll
    for (int n = 0; n < kScanRungs; ++n) {
        n_reach += (A.scan.r[n] <= i0 + kTile - 1) ? 1 : 0;
        n_lo += (A.scan.a[n] <= kNear - (INT ? 0 : 1)) ? 1 : 0;
    }
    // near rungs: the prefix with a <= 63 (near and far rows inside the near block; INT: a <= 64,
    // the one row). Steps k < kn come from the near block, kn even: rung pairs 2k, 2k + 1, or (INT)
    // for even k a group of the four rungs 2k .. 2k + 3 (those past nn are padding). Steps kn ..
    // n_steps - 1 are far steps, step k in buffer (k + 1) % 2, holding rungs 2k - ro and
    // 2k - ro + 1 (ro = 0 unless INT).
    const int n_near = min(n_lo, n_reach);
    const int nn = INT ? min(n_near, 8) : 0;
    const int kn = INT ? 2 * ((nn + 3) >> 2) : (n_near >> 1) & ~1;
    const int ro = INT ? 2 * kn - nn : 0;
    const int n_steps = INT ? kn + ((n_reach - nn + 1) >> 1) : (n_reach + 1) >> 1;
    constexpr int kStepDmas = INT ? 4 : 6;              // DMA instructions per wave of a far step

    const int64_t kv_row0 = static_cast<int64_t>(bg) * L;
    const __amdgpu_buffer_rsrc_t krs = rows_rsrc(A.kstage, kv_row0, L);
    const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(A.vstage, kv_row0, L);
    Stager st;
    st.init(lane, wave);
    // rung step k: rungs 2k and 2k + 1 (zeros past the reach); the far row of position p sits at
    // slot p (block A) or 72 + p + 2 (block B), the near row one slot up
    // (INT: the near row of position p at slot p or 72 + p)
    auto step = [&](const __amdgpu_buffer_rsrc_t& rs, char* dst, int k) {
        if constexpr (INT) {
            const int n = 2 * k - ro;
            st.step64(rs, dst, n < n_reach, i0 - A.off[n].a, n + 1 < n_reach, i0 - A.off[n + 1].a);
        } else {
            st.step(rs, dst, 2 * k < n_reach, i0 - A.off[2 * k].a - 1, 2 * k + 1 < n_reach, i0 - A.off[2 * k + 1].a - 3);
        }
    };
    const int jn = i0 - kNear;                          // the near block's row at slot 0
    auto buf = [&](int j) -> char* { return (j & 1) ? lds1 : lds0; };

    // ---- prologue: q of the lane's row (head h0 + x, position i; past L the row L - 1, finite
    // and never used) straight into registers, 16 bytes at a time, then the key near block (item
    // 0) and item 1 (key far step kn): all in flight together, and the q build below waits for q
    // alone (loads count in vmcnt in issue order) ----
    uint4 qraw[8];
    float4 ctab[4];
    uint32_t flagged;                                   // nonzero: a staged row the lane checks lies outside fp16's range
    {
        const uint4* qrow = reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(A.q) +
                                                           ((static_cast<int64_t>(b) * A.Hq + h0 + x) * L + min(i, L - 1)) * kD);
#pragma unroll
        for (int c = 0; c < 8; ++c) qraw[c] = qrow[c];
        // the cos/sin of the position: lane x loads pairs 8x..8x+7; the rotation takes the others
        // from the quad's lanes
        const float4* ct = reinterpret_cast<const float4*>(A.cstab) + static_cast<int64_t>(active ? i : 0) * (kPairs / 2) + 4 * x;
#pragma unroll
        for (int u = 0; u < 4; ++u) ctab[u] = ct[u];
        // the range flags of the staged rows this tile reads
        flagged = rows_flagged(A, bg / kPrepRowGroup, i0, n_reach);
    }
    st.near(krs, lds0, jn);
    step(krs, lds1, kn);                                // (zero rows when no far rung is reached)
    // whether some row of the tile lies outside the fp16 range (then the whole tile is computed in
    // float32): each wave's vote, read after a later barrier
    post_vote(votes, wave, flagged != 0u || (active && q_outside_fp16(qraw, A.qscale)));

    // q of head h0 + x, rotated at its position and scaled by qscale, fp16, in the keys' permuted
    // order: word 2m holds dims (m, 16 + m), word 2m + 1 dims (32 + m, 48 + m), i.e. the x and y
    // halves of RoPE pairs m and 16 + m; register chunk c = words 4c..4c+3
    uint32_t q[8][4];
    {
        auto dim = [&](int d) -> float {               // bf16 dim d of the raw row
            const uint4& r = qraw[d >> 3];
            const int w = (d >> 1) & 3;
            const uint32_t v = w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
            return (d & 1) ? bf16_hi(v) : bf16_lo(v);
        };
        auto cos_sin = [&](int pair) -> float2 {         // pair: compile-time; from lane pair >> 3
            const float4& t = ctab[(pair & 7) >> 1];
            const float c = (pair & 1) ? t.z : t.x, sn = (pair & 1) ? t.w : t.y;
            switch (pair >> 3) {
                case 0: return make_float2(quad_f<kBcast0>(c), quad_f<kBcast0>(sn));
                case 1: return make_float2(quad_f<kBcast1>(c), quad_f<kBcast1>(sn));
                case 2: return make_float2(quad_f<kBcast2>(c), quad_f<kBcast2>(sn));
                default: return make_float2(quad_f<kBcast3>(c), quad_f<kBcast3>(sn));
            }
        };
        const float qs = A.qscale;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            const float2 t0 = cos_sin(m), t1 = cos_sin(16 + m);
            const float x0 = dim(m), y0 = dim(32 + m), x1 = dim(16 + m), y1 = dim(48 + m);
            q[m >> 1][2 * (m & 1)] = pack_h2((x0 * t0.x - y0 * t0.y) * qs, (x1 * t1.x - y1 * t1.y) * qs);
            q[m >> 1][2 * (m & 1) + 1] = pack_h2((y0 * t0.x + x0 * t0.y) * qs, (y1 * t1.x + x1 * t1.y) * qs);
        }
    }
    publish<kStepDmas>();                               // the key near block has landed
    clk.mark(1);

    // ---- phase A: scores of the lane's head x (base 2) ----
    // Far step k computes from buffer (k + 1) % 2 after issuing step k + 1 into the other buffer
    // (the barrier that ended the item before released it); the wait before each barrier is for
    // step k + 1, the only load in flight.
    float s[4 * kWG + MAXK];
    // lane x of a rung group: rung 2k + (x >> 1), near (x even) or far row (INT: the near rows of
    // rungs 2k - ro and 2k - ro + 1 in columns 0 and 2); the scores go to slots 2k and 2k + 1
    auto score = [&](const f4_t& acc, int k) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int n = 2 * k + e - ro;
            if (n < n_reach) {
                const float sc = INT ? acc[2 * e] : fmaf(A.off[n].t, acc[2 * e + 1] - acc[2 * e], acc[2 * e]);
                s[4 * kWG + 2 * k + e] = (active && i >= A.off[n].a + A.off[n].interp) ? sc : kNegInf;
            }
        }
    };
    // INT, near group of step k (even): the distance of rung 2k + c, 0 (the window's own row, a
    // staged row) for padding
    auto near_a = [&](int k, int c) -> int { return 2 * k + c < nn ? A.off[2 * k + c].a : 0; };
    {
        // item 0: lane x reads window distance d = 4g + x, slot p - d + 64 (pads d > W read
        // staged rows); then the near rung pairs: rung 2k + (x >> 1), near row i - a at slot
        // p + 64 - a (x even) or far row one slot down
        const int s0 = p - x + kNear;
#pragma unroll
        for (int g = 0; g < kWG; ++g) {
            f4_t acc = {0.f, 0.f, 0.f, 0.f};
            if (4 * g <= W) acc = row_dot_group(q, buf(0), (s0 - 4 * g) * kRowBytes, swz(s0 - 4 * g));
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 4 * g + r;
                s[d] = (active && d <= W && i >= d) ? acc[r] : kNegInf;
            }
        }
#pragma unroll
        for (int y = 4 * kWG; y < 4 * kWG + MAXK; ++y) s[y] = kNegInf;
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if constexpr (INT) {
                // lane x reads rung 2k + x, row i - a at slot p + 64 - a
                if ((k & 1) == 0 && k < kn) {
                    const int sl = p + kNear - pick4(x, near_a(k, 0), near_a(k, 1), near_a(k, 2), near_a(k, 3));
                    const f4_t acc = row_dot_group(q, buf(0), sl * kRowBytes, swz(sl));
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int n = 2 * k + c;
                        if (n < nn) s[4 * kWG + n] = (active && i >= A.off[n].a) ? acc[c] : kNegInf;
                    }
                }
            } else if (k < kn) {
                const int sl = p + kNear - pick_uniform((x >> 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a) - (x & 1);
                score(row_dot_group(q, buf(0), sl * kRowBytes, swz(sl)), k);
            }
        }
        publish<0>();                                   // item 1 has landed, buffer 0 is free
    }
    // far steps: lane x reads rung 2k + (x >> 1), near (x even) or far row (INT: the near row,
    // for x even and odd alike)
    const int rslot = INT ? p + ((x >> 1) ? kBlkSlots : 0) : p + ((x >> 1) ? kBlkSlots + 2 : 0) + ((x & 1) ? 0 : 1);
    const int rbase = rslot * kRowBytes, rsw = swz(rslot);
    // The last far step computes from buffer 1 when there is an odd number of them (kn is even):
    // buffer 0 is free then, and the value near block goes ahead under that step (its barrier
    // waits for the step's loads only: the near block's 4 transfers per wave stay in flight).
    const bool near_ahead = n_steps > kn && ((n_steps - kn) & 1) != 0;
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        if (k >= kn && k < n_steps) {                   // buffer (k + 1) % 2
            const bool last = k + 1 >= n_steps;
            if (!last) step(krs, buf(k + 2), k + 1);
            else if ((k & 1) == 0) st.near(vrs, lds0, jn);
            score(row_dot_group(q, buf(k + 1), rbase, rsw), k);
            if (last && (k & 1) == 0)
                publish<4>();
            else
                publish<0>();
        }
    }

    clk.mark(2);
    // ---- value near block into buffer 0 (unless it went ahead) and value far step kn into
    // buffer 1 (both free after the last barrier), under the softmax ----
    if (!near_ahead) st.near(vrs, lds0, jn);
    step(vrs, lds1, kn);

    // ---- exact softmax; weights as fp16 groups of 4 ----
    float m = kNegInf;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) m = fmaxf(m, s[y]);
    if (!active) m = 0.f;
    float l = 0.f;
#pragma unroll
    for (int y = 0; y < 4 * kWG + MAXK; ++y) {
        s[y] = __builtin_amdgcn_exp2f(s[y] - m);   // v_exp_f32; s - m <= 0
        l += s[y];
    }
    asm volatile("" : "+v"(l));                     // the sum now: the exponentials die with the packing
    uint32_t pw[kWG][2], po[MAXS][2];
#pragma unroll
    for (int g = 0; g < kWG; ++g) {
        pw[g][0] = pack_h2(s[4 * g], s[4 * g + 1]);
        pw[g][1] = pack_h2(s[4 * g + 2], s[4 * g + 3]);
    }
#pragma unroll
    for (int k = 0; k < MAXS; ++k) {
        if constexpr (INT) {
            // a near group (even k < kn): slots 2k .. 2k + 3, one row each; a far step: the near
            // rows of its two rungs in group slots 0 and 2 (slots 1 and 3 weigh 0)
            auto ev = [&](int y) { return y < MAXK ? s[4 * kWG + y] : 0.f; };
            const bool grp = k < kn && (k & 1) == 0;
            po[k][0] = pack_h2(ev(2 * k), grp ? ev(2 * k + 1) : 0.f);
            po[k][1] = grp ? pack_h2(ev(2 * k + 2), ev(2 * k + 3)) : pack_h2(ev(2 * k + 1), 0.f);
        } else {
            float w[4];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int n = 2 * k + e;
                const float ev = s[4 * kWG + n];
                const float far = (n < n_reach) ? ev * A.off[n].t : 0.f;   // ev is 0 past the reach
                w[2 * e] = ev - far;
                w[2 * e + 1] = far;
            }
            po[k][0] = pack_h2(w[0], w[1]);
            po[k][1] = pack_h2(w[2], w[3]);
        }
    }

    // ---- phase B: P.V ----
    // The B operand of dim block m for lane (p', x) is (v[row 0][16x + m], .., v[row 3][16x + m]).
    // ds_read_b64_tr_b16 transposes within each 16 lanes: lane (p', x) receives element x of the
    // 8 bytes that lane (4 (p' >> 2) + k, p' & 3) read, for k = 0..3. So lane (p', x) reads, for
    // position pt = 4 (p' >> 2) + x of the wave and slot k = p' & 3 of the group, elements
    // 4m..4m+3 of that row: dims 16c + m, c = 0..3.
    const int pt = 16 * wave + 4 * (pq >> 2) + x;       // the position this lane reads for
    const int kt = pq & 3;                              // the slot of the group this lane reads
    f4_t o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (f4_t){0.f, 0.f, 0.f, 0.f};
    {
        publish<kStepDmas>();                           // the value near block has landed
        clk.mark(3);
        // window group g: slot pt - 4g - kt + 64
        const int sv = pt - kt + kNear;
#pragma unroll
        for (int g = 0; g < kWG; ++g)
            if (4 * g <= W) row_sum_group(o, pw[g][0], pw[g][1], lds0, (sv - 4 * g) * kRowBytes, swz(sv - 4 * g));
        // near rung pairs: slot kt of the group is rung 2k + (kt >> 1), near row pt - a at slot
        // pt + 64 - a (kt even) or far row one slot down
        // (INT: slot kt of the group is rung 2k + kt, for even k)
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if constexpr (INT) {
                if ((k & 1) == 0 && k < kn) {
                    const int sl = pt + kNear - pick4(kt, near_a(k, 0), near_a(k, 1), near_a(k, 2), near_a(k, 3));
                    row_sum_group(o, po[k][0], po[k][1], lds0, sl * kRowBytes, swz(sl));
                }
            } else if (k < kn) {
                const int sl = pt + kNear - pick_uniform((kt >> 1) != 0, A.off[2 * k + 1].a, A.off[2 * k].a) - (kt & 1);
                row_sum_group(o, po[k][0], po[k][1], lds0, sl * kRowBytes, swz(sl));
            }
        }
        if (n_steps > kn) publish<0>();                 // value far step kn has landed, buffer 0 is free
    }
    {
        // slot k of a far step's group: near and far of rung 2k (block A, slots pt + 1, pt) and
        // of rung 2k + 1 (block B, slots pt + 3, pt + 2) (INT: the near rows, slots pt and
        // 72 + pt, each read twice); value step k sits in buffer (k + 1) % 2
        const int sv = INT ? pt + ((kt < 2) ? 0 : kBlkSlots) : (kt < 2) ? pt + 1 - kt : kBlkSlots + pt + 5 - kt;
        const int vbase = sv * kRowBytes, vsw = swz(sv);
#pragma unroll
        for (int k = 0; k < MAXS; ++k) {
            if (k >= kn && k < n_steps) {
                if (k + 1 < n_steps) step(vrs, buf(k + 2), k + 1);
                row_sum_group(o, po[k][0], po[k][1], buf(k + 1), vbase, vsw);
                if (k + 1 < n_steps) publish<0>();
            }
        }
    }

    clk.mark(4);
    // ---- normalise and write: lane x holds dims 16x..16x+15 of heads 0..3 ----
    const float inv = 1.0f / l;
    float invh[4];
    invh[0] = quad_f<kBcast0>(inv);
    invh[1] = quad_f<kBcast1>(inv);
    invh[2] = quad_f<kBcast2>(inv);
    invh[3] = quad_f<kBcast3>(inv);
    const int outside = or_votes(votes);                // (posted before the first publish)
    if (active && !outside) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bf16_t* orow = static_cast<bf16_t*>(A.o) + ((static_cast<int64_t>(b) * A.Hq + h0 + r) * L + i) * kD + 16 * x;
            uint4 lo, hi;
            lo.x = pack_bf2(o[0][r] * invh[r], o[1][r] * invh[r]);
            lo.y = pack_bf2(o[2][r] * invh[r], o[3][r] * invh[r]);
            lo.z = pack_bf2(o[4][r] * invh[r], o[5][r] * invh[r]);
            lo.w = pack_bf2(o[6][r] * invh[r], o[7][r] * invh[r]);
            hi.x = pack_bf2(o[8][r] * invh[r], o[9][r] * invh[r]);
            hi.y = pack_bf2(o[10][r] * invh[r], o[11][r] * invh[r]);
            hi.z = pack_bf2(o[12][r] * invh[r], o[13][r] * invh[r]);
            hi.w = pack_bf2(o[14][r] * invh[r], o[15][r] * invh[r]);
            store_nt(orow, lo);
            store_nt(orow + 8, hi);
        }
        if (A.lse != nullptr)
            store_nt(A.lse + (static_cast<int64_t>(b) * A.Hq + h0 + x) * L + i, (m + log2f(l)) * 0.69314718055994530942f);
    }
    if (outside) {
        // Some row of the tile lies outside fp16's range: what the matrix cores computed is not
        // stored, and the tile is computed in float32 from the caller's rows instead (here at the
        // end, where nothing of the matrix-core path is live: the fallback's registers are its own).
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        fwd_tile_fp32(A, b, bg, h0, i0);
    }
    clk.record(tile, n_steps, kn, n_reach);
}

}  // namespace

hipError_t launch_prep_kv16(const PrepArgs& A, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(A.n_blk), static_cast<unsigned>((A.n_bh + kPrepRows - 1) / kPrepRows));
    if (A.main && A.k16lo != nullptr)
        hipLaunchKernelGGL((prep_kv16_kernel<true, true>), grid, dim3(256), 0, s, A);
    else if (A.main)
        hipLaunchKernelGGL((prep_kv16_kernel<true, false>), grid, dim3(256), 0, s, A);
    else if (A.k16lo != nullptr)
        hipLaunchKernelGGL((prep_kv16_kernel<false, true>), grid, dim3(256), 0, s, A);
    return hipGetLastError();
}

bool fwd_mfma_supported(const FwdArgs& A) {
    return A.G % 4 == 0 && A.W <= 15 && A.n_off <= 16;
}

hipError_t launch_fwd_mfma(const FwdArgs& A0, hipStream_t s) {
    FwdArgs A = A0;
    const int64_t n_tiles = (A.L + kTile - 1) / kTile;
    const int64_t n_units = static_cast<int64_t>(A.B) * A.Hkv * (A.G / 4);
    // the forward keeps 4 workgroups per CU in one round: mix early and late tiles on each CU
    A.xcd_map = (n_units % 8 == 0) ? 2 : 0;
    const dim3 grid(static_cast<unsigned>(n_units * n_tiles));
    if (int_path_fits(A.off, A.n_off, 8))
        hipLaunchKernelGGL((fwd_mfma_kernel<8, true>), grid, dim3(kNT), 0, s, A);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<8, false>), grid, dim3(kNT), 0, s, A);
    return hipGetLastError();
}

}  // namespace fibattn

extern "C" fibattn_status_t fibattn_phase_trace_read(uint64_t* out, int32_t n_wg) {
#ifdef FIBATTN_PHASE_TRACE
    if (out == nullptr || n_wg < 0 || n_wg > fibattn::kTraceWgs)
        return static_cast<fibattn_status_t>(
            fibattn::report_error(FIBATTN_ERR_INVALID, "phase trace: out is null or n_wg = %d outside 0..%d", n_wg,
                                  fibattn::kTraceWgs));
    const hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(fibattn::g_phase),
                                             static_cast<size_t>(n_wg) * fibattn::kTraceWords * sizeof(uint64_t));
    if (e != hipSuccess)
        return static_cast<fibattn_status_t>(
            fibattn::report_error(FIBATTN_ERR_HIP, "phase trace: %s", hipGetErrorString(e)));
    return FIBATTN_OK;
#else
    (void)out;
    (void)n_wg;
    return static_cast<fibattn_status_t>(
        fibattn::report_error(FIBATTN_ERR_UNSUPPORTED, "this library was built without the phase trace"));
#endif
}
