// Matrix-core building blocks shared by the gfx950 forward and backward kernels for bfloat16
// storage: 4x4x4 fp16 MFMA groups, the LDS slot swizzle, the transposing LDS read, LDS DMA staging
// of shifted row blocks with counted waits. Included by the .hip files only.
//
// Layout conventions (section references: "Depth-Staggered Fibonacci Spacing for Sparse
// Attention", §2 "Attended set"):
//  * A workgroup owns 64 consecutive positions of one (batch, key-value head) and 4 query heads;
//    wave w takes positions 16w..16w+15, lane 4p' + x is position p' of the wave and head (or
//    slot, or dim column) x. v_mfma_f32_4x4x4_16b_f16 computes one 4x4x4 block per position:
//    lane 4p' + x is row x of A and column x of B and of the result, of block p'.
//  * A group is 4 virtual slots: 4 window distances, or (near, far) of two consecutive rungs. An
//    interpolated rung reads two rows, nearer (coefficient 1 - t) and farther (t); scores and
//    outputs are linear in the blended row.
//  * LDS slots are 128-byte fp16 rows; 16-byte chunk k of slot s sits at chunk k ^ ((s >> 1) & 7).
//    A far step holds rung 2k at slot 0 (block A) and rung 2k + 1 at slot kBlkSlots (block B,
//    two slots up); a near block holds 128 consecutive rows, row j0 + s at slot s.
#pragma once

#include "fibattn_device.h"

namespace fibattn {
namespace mx {

constexpr int kNT = 256;                 // 4 waves x 16 positions x 4 lanes
constexpr int kRowBytes = kD * 2;        // one fp16 row
constexpr int kBlkSlots = 72;            // 65 (+2 for the second rung) rows, 9 DMA groups
constexpr int kBlkBytes = kBlkSlots * kRowBytes;
constexpr int kBufBytes = 2 * kBlkBytes; // one staging buffer: a near block or a far step
// The near block of a tile of 64 positions i0..i0+63: key rows i0 - 64 .. i0 + 63 (slot s holds
// row i0 - kNear + s). It holds the window (W <= 15) and both rows of every rung with a <= 63.
constexpr int kNear = 64;
constexpr int kWG = 4;                   // window groups (W <= 15)
constexpr int kBcast0 = 0x00, kBcast1 = 0x55, kBcast2 = 0xAA, kBcast3 = 0xFF;   // quad_perm [r,r,r,r]
constexpr int kXor2 = 0x4E;              // quad_perm [2,3,0,1]: lane x ^ 2
constexpr int kPerm0202 = 0x88;          // quad_perm [0,2,0,2]: lane 2 (x & 1)
constexpr int kPerm1313 = 0xDD;          // quad_perm [1,3,1,3]: lane 2 (x & 1) + 1
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, gfx9 family

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ f4_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f4_t c) {
    return __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, (u2_t){a0, a1}),
                                              __builtin_bit_cast(h4_t, (u2_t){b0, b1}), c, 0, 0, 0);
}

template <int CTRL> __device__ __forceinline__ float quad_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// The 4 floats of lane c (compile-time) of the quad, in every lane of the quad.
__device__ __forceinline__ float4 quad_bcast(int c, const float4& v) {
    switch (c) {
        case 0: return make_float4(quad_f<kBcast0>(v.x), quad_f<kBcast0>(v.y), quad_f<kBcast0>(v.z), quad_f<kBcast0>(v.w));
        case 1: return make_float4(quad_f<kBcast1>(v.x), quad_f<kBcast1>(v.y), quad_f<kBcast1>(v.z), quad_f<kBcast1>(v.w));
        case 2: return make_float4(quad_f<kBcast2>(v.x), quad_f<kBcast2>(v.y), quad_f<kBcast2>(v.z), quad_f<kBcast2>(v.w));
        default: return make_float4(quad_f<kBcast3>(v.x), quad_f<kBcast3>(v.y), quad_f<kBcast3>(v.z), quad_f<kBcast3>(v.w));
    }
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    const h2_t v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// Two floats as bfloat16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
    typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
    typedef float fl2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((fl2_t){lo, hi}, bf2_t));
}

__device__ __forceinline__ uint4 lds16(const char* lds, int addr) {
    return *reinterpret_cast<const uint4*>(lds + addr);
}

// The chunk swizzle of slot s, as a byte offset to XOR into (logical chunk << 4).
__device__ __forceinline__ int swz(int s) { return ((s >> 1) & 7) << 4; }

// An LDS DMA destination passed through an opaque (uniform) value: the compiler then keeps no
// record of which LDS array a DMA writes and adds no waits of its own before LDS reads;
// publish<N> orders every read after the DMA it needs.
__device__ __forceinline__ lds_ptr_t dma_dst(char* dst) {
    uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)dst));
    asm volatile("" : "+s"(a));   // an SGPR: the value is the same for the whole wave
    return (lds_ptr_t)static_cast<uintptr_t>(a);
}

// A per-lane choice between two uniform values (two entries of the kernel's offset table): both
// are read as scalars first, each made opaque in a scalar register, and the lane then selects
// (v_cndmask). A choice between the table entries themselves would become one vector load from a
// per-lane kernel-argument address, which the compiler follows with a full vmcnt wait behind
// every staging load in flight; an empty asm inside each arm of the choice would become a branch.
template <typename T> __device__ __forceinline__ T pick_uniform(bool c, T if_true, T if_false) {
    asm volatile("" : "+s"(if_true));
    asm volatile("" : "+s"(if_false));
    return c ? if_true : if_false;
}

// pick_uniform among four: lane choice c (0..3) of four uniform values.
template <typename T> __device__ __forceinline__ T pick4(int c, T v0, T v1, T v2, T v3) {
    asm volatile("" : "+s"(v0));
    asm volatile("" : "+s"(v1));
    asm volatile("" : "+s"(v2));
    asm volatile("" : "+s"(v3));
    const T lo = (c & 1) ? v1 : v0, hi = (c & 1) ? v3 : v2;
    return (c & 2) ? hi : lo;
}

// Whether a plan takes the integer-offset kernels: every kept rung integral, and the steps of a
// tile that reaches every rung fit in maxs: the rungs with a <= 64 (at most 8) come from the near
// block four to a group (two steps per group), the others two to a far step. (The count only
// grows with the rungs a tile reaches.)
inline bool int_path_fits(const OffsetSlot* off, int n_off, int maxs) {
    if (n_off == 0) return false;
    int n_near = 0;
    for (int n = 0; n < n_off; ++n) {
        if (off[n].interp) return false;
        if (off[n].a <= kNear) n_near = n + 1;
    }
    const int nn = n_near < 8 ? n_near : 8;
    return 2 * ((nn + 3) / 4) + (n_off - nn + 1) / 2 <= maxs;
}

// Wait until at most N vector-memory instructions of this wave are in flight (its LDS DMAs up to
// the block the next step reads have landed) and its LDS reads are done, then the workgroup
// barrier. __syncthreads would also drain every staging load in flight.
template <int N> __device__ __forceinline__ void publish() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Product of one group with a per-head operand x held in registers (register chunk c = elements
// 8c..8c+7 of the staged row order): lane x supplies the row at slot byte offset base (swizzle
// F = swz(slot)), x supplies head x; returns head x's 4 products. Four accumulators keep the
// dependent chains short.
__device__ __forceinline__ f4_t row_dot_group(const uint32_t (&x)[8][4], const char* lds, int base, int F) {
    f4_t a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = (f4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint4 k = lds16(lds, base | ((c << 4) ^ F));
        a[(2 * c) & 3] = mfma4(k.x, k.y, x[c][0], x[c][1], a[(2 * c) & 3]);
        a[(2 * c + 1) & 3] = mfma4(k.z, k.w, x[c][2], x[c][3], a[(2 * c + 1) & 3]);
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// row_dot_group with both operands split into a high and a low fp16 part (x = xh + xl, the staged
// rows = hi + lo): xh.hi + xl.hi + xh.lo, the product to about 2^-22 relative (xl.lo is below
// that). The two staged halves sit at the same slot offset of lds_hi and lds_lo.
__device__ __forceinline__ f4_t row_dot_group_x3(const uint32_t (&xh)[8][4], const uint32_t (&xl)[8][4],
                                                 const char* lds_hi, const char* lds_lo, int base, int F) {
    f4_t a[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = (f4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int addr = base | ((c << 4) ^ F);
        const uint4 k = lds16(lds_hi, addr);
        const uint4 kl = lds16(lds_lo, addr);
        a[(2 * c) & 3] = mfma4(k.x, k.y, xh[c][0], xh[c][1], a[(2 * c) & 3]);
        a[(2 * c + 1) & 3] = mfma4(k.z, k.w, xh[c][2], xh[c][3], a[(2 * c + 1) & 3]);
        a[(2 * c) & 3] = mfma4(k.x, k.y, xl[c][0], xl[c][1], a[(2 * c) & 3]);
        a[(2 * c + 1) & 3] = mfma4(k.z, k.w, xl[c][2], xl[c][3], a[(2 * c + 1) & 3]);
        a[(2 * c) & 3] = mfma4(kl.x, kl.y, xh[c][0], xh[c][1], a[(2 * c) & 3]);
        a[(2 * c + 1) & 3] = mfma4(kl.z, kl.w, xh[c][2], xh[c][3], a[(2 * c + 1) & 3]);
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// ds_read_b64_tr_b16 at lds + addr: 4 fp16 (or bf16) elements, as a whole. (Splitting the result
// into its two dwords is left to the callers that need it: an optimisation has been seen to fold
// the second dword of this builtin's result onto the first.)
__device__ __forceinline__ h4_t tr_read_h4(const char* lds, int addr) {
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4_t* lds_s4_t;
    return __builtin_bit_cast(h4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4_t)(lds + addr)));
}

// Weighted sum of one group's rows. The lane reads its assigned (position, slot) row, at slot
// byte offset base with swizzle F, for element blocks m = 0..15 (elements 4m..4m+3: byte 8m of
// the staged row). ds_read_b64_tr_b16 transposes within each 16 lanes and hands every lane the 4
// rows' element 4m + x; (w01, w23) are the lane's head's weights, o[m] accumulates element
// 4m + x of the 4 heads.
__device__ __forceinline__ void row_sum_group(f4_t (&o)[16], uint32_t w01, uint32_t w23, const char* lds, int base,
                                              int F) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
        const int addr = (base | (((m >> 1) << 4) ^ F)) + 8 * (m & 1);
        o[m] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, (u2_t){w01, w23}), tr_read_h4(lds, addr), o[m],
                                                  0, 0, 0);
    }
}

// LDS DMA staging of one (batch, kv head)'s fp16 rows. A 16-byte wave instruction fills 1 KB = 8
// slots: lane l lands on slot 8g + (l >> 3), physical chunk l & 7, and fetches that slot's row and
// the logical chunk the swizzle puts there. A 4-byte instruction fills 2 slots: lane l lands on
// slot 2g' + (l >> 5), physical dword l & 31. Every wave issues the same number of instructions
// per item (4 per near block, 3 per rung block), so the waits can count them. Rows before 0 or
// past L fall outside the buffer resource and arrive as zeros.
// Blocks are given by the row that lands at slot 0. (Rows are passed by value: taking the address
// of the kernel's argument struct would make the compiler copy it to scratch memory.)
struct Stager {
    int wave, gpar;
    int voff16_0, voff16_1, voff4_0, voff4_1;   // per swizzle parity / block (no indexed arrays:
                                                // those would put the struct in scratch memory)

    __device__ __forceinline__ void init(int lane, int wave_) {
        wave = wave_;
        gpar = wave & 1;                                // parity of this wave's groups in block A
        // 16-byte part: slot 8g + lrow has swizzle (4 (g & 1) + (lrow >> 1)) & 7, per parity of g
        const int lrow = lane >> 3;
        voff16_0 = lrow * kRowBytes + (((lane & 7) ^ (lrow >> 1)) << 4);
        voff16_1 = lrow * kRowBytes + (((lane & 7) ^ (4 + (lrow >> 1))) << 4);
        // 4-byte part: slot 64 + 2 wave + (lane >> 5) (block B: 72 more) has swizzle wave (4 + wave)
        const int dw = lane & 31;
        voff4_0 = (lane >> 5) * kRowBytes + (((dw >> 2) ^ wave) << 4) + ((dw & 3) << 2);
        voff4_1 = (lane >> 5) * kRowBytes + (((dw >> 2) ^ (4 + wave)) << 4) + ((dw & 3) << 2);
    }
    __device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t& rs, char* dst, int row0, int par) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dma_dst(dst), 16, row0 * kRowBytes + (par ? voff16_1 : voff16_0), 0, 0, 0);
    }
    __device__ __forceinline__ void dma4(const __amdgpu_buffer_rsrc_t& rs, char* dst, int row0, int blk) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dma_dst(dst), 4, row0 * kRowBytes + (blk ? voff4_1 : voff4_0), 0, 0, 0);
    }
    // near block: rows j0 + s at slot s, s < 128 (16 groups, 4 per wave)
    __device__ __forceinline__ void near(const __amdgpu_buffer_rsrc_t& rs, char* dst, int j0) const {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int g = wave + 4 * u;
            dma16(rs, dst + g * 1024, j0 + 8 * g, gpar);
        }
    }
    // rung block blk (0: A, 1: B at slot 72): rows j0 + s at slot s < 72; two 16-byte groups and
    // one 4-byte pair per wave (block B starts at slot 72 = 9 groups: its groups have the other
    // parity). A block that is not real stages rows before 0: zeros.
    __device__ __forceinline__ void rung(const __amdgpu_buffer_rsrc_t& rs, char* dst, bool real, int j0_real,
                                         int blk) const {
        const int j0 = real ? j0_real : -(kTile + kBlkSlots + 8);
        dma16(rs, dst + wave * 1024, j0 + 8 * wave, gpar ^ blk);
        dma16(rs, dst + (wave + 4) * 1024, j0 + 8 * (wave + 4), gpar ^ blk);
        dma4(rs, dst + 64 * kRowBytes + wave * 256, j0 + 64 + 2 * wave, blk);
    }
    // a rung block of 64 rows (integral rungs: no second row), slots 0..63 of the block
    __device__ __forceinline__ void rung64(const __amdgpu_buffer_rsrc_t& rs, char* dst, bool real, int j0_real,
                                           int blk) const {
        const int j0 = real ? j0_real : -(kTile + kBlkSlots + 8);
        dma16(rs, dst + wave * 1024, j0 + 8 * wave, gpar ^ blk);
        dma16(rs, dst + (wave + 4) * 1024, j0 + 8 * (wave + 4), gpar ^ blk);
    }
    __device__ __forceinline__ void step64(const __amdgpu_buffer_rsrc_t& rs, char* dst, bool r0, int j0a, bool r1,
                                           int j0b) const {
        rung64(rs, dst, r0, j0a, 0);
        rung64(rs, dst + kBlkBytes, r1, j0b, 1);
    }
    // a rung step: block A from row j0a, block B from row j0b
    __device__ __forceinline__ void step(const __amdgpu_buffer_rsrc_t& rs, char* dst, bool r0, int j0a, bool r1,
                                         int j0b) const {
        rung(rs, dst, r0, j0a, 0);
        rung(rs, dst + kBlkBytes, r1, j0b, 1);
    }
};

// Wave-private LDS transposes between the lanes' rows and contiguous memory. In the row view lane
// (p', x) holds the 128-byte row of head x at position p' of the wave as 8 chunks; the row's slot
// in the wave's 8 KB region is s = 16 x + p' (head-major: a head's 16 positions are 2 KB of
// contiguous memory). In the linear view, instruction u (0..7) covers slots 8u..8u+7: lane l
// holds chunk l & 7 of slot 8u + (l >> 3), so a wave's global access is 1 KB of contiguous rows.
// Chunk c of slot s sits at chunk c ^ tr_f(s); a pass of 16 lanes then touches 16 distinct banks
// in both views.
__device__ __forceinline__ int tr_f(int s) { return ((s >> 1) & 1) | ((s >> 4) << 1); }
__device__ __forceinline__ int row_view_addr(int pq, int x, int c) {
    const int s = 16 * x + pq;
    return s * kRowBytes + ((c ^ tr_f(s)) << 4);
}
__device__ __forceinline__ int lin_view_addr(int lane, int u) {
    const int s = 8 * u + (lane >> 3);
    return s * kRowBytes + (((lane & 7) ^ tr_f(s)) << 4);
}
// the slot (head-major) of linear-view instruction u for this lane
__device__ __forceinline__ int lin_slot(int lane, int u) { return 8 * u + (lane >> 3); }

// Buffer resource over rows [row0, row0 + L) of 128-byte rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int64_t row0, int L) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(static_cast<const char*>(base) + row0 * kRowBytes), 0,
                                             L * kRowBytes, kRsrcWord3);
}

// Workgroup -> (unit, tile): with the XCD map (xcd_map != 0), unit u runs on XCD u % 8 for all its
// tiles, whose L2 then holds that unit's keys and values for every tile that re-reads them. An XCD
// hands its workgroups (slot s = w / 8 in launch order) to its 32 CUs in turn, so slots s, s + 32,
// s + 64, ... share a CU. With xcd_map == 2, every odd row of 32 slots is taken in reverse order,
// so that a CU holds early tiles (few rungs in reach) and late ones alike instead of four copies of
// one tile index; a partial last row keeps its order (the map stays a permutation).
// With xcd_map == 3 (units per XCD a multiple of 4) an XCD takes its units four at a time, and
// the slots of a group of four run tile-major: tile 0 of the four units, then tile 1, ... The key
// kernel takes it. A low key tile is read by the most rungs, so the group's longest workgroups
// start first and the light ones fill in behind them, while the four units' rows that the group
// re-reads still fit the XCD's L2 (two workgroups per CU: 64 slots, four units of 16 tiles at
// L = 1024). Measured at B = 32, L = 1024: 81.3 -> 76.8 us with unchanged HBM bytes; tile-major
// over all eight units was about as fast but fetched 13 % more.
__device__ __forceinline__ void unit_tile(int w, int n_tiles, int xcd_map, int& unit, int& tile) {
    if (xcd_map == 3) {
        const int sl = w >> 3, grp = sl / (4 * n_tiles), r = sl % (4 * n_tiles);
        tile = r >> 2;
        unit = (4 * grp + (r & 3)) * 8 + (w & 7);
        return;
    }
    if (xcd_map) {
        int sl = w >> 3;
        const int row = sl >> 5;
        if (xcd_map == 2 && (row & 1) && ((row + 1) << 5) <= static_cast<int>(gridDim.x >> 3))
            sl = (row << 5) + 31 - (sl & 31);
        unit = (sl / n_tiles) * 8 + (w & 7);
        tile = sl % n_tiles;
    } else {
        unit = w / n_tiles;
        tile = w % n_tiles;
    }
}

// ---- rows outside fp16's range, and the float32 tiles that take them ----
// fp16 holds a row exactly enough only inside a range: every element below 2^15 in magnitude
// (65504 is fp16's largest) and, unless the row is zero, a row maximum of at least 2^-10 (below
// that the row's largest elements come near fp16's subnormals, 2^-14, where relative precision is
// lost).
constexpr float kFp16Big = 32768.0f;               // 2^15
constexpr float kFp16Small = 0.0009765625f;        // 2^-10

// The bits of the largest magnitude among a row's 64 bf16 values (15 bits, sign cleared): bf16
// magnitudes order as unsigned integers, so packed 16-bit maxima find it without a conversion.
__device__ __forceinline__ uint32_t max_abs_bf16_bits(const uint4 (&r)[8]) {
    typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
    u16x2_t m[4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t w[4] = {r[c].x, r[c].y, r[c].z, r[c].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const u16x2_t v = __builtin_bit_cast(u16x2_t, w[e] & 0x7fff7fffu);
            m[e] = (c == 0) ? v : __builtin_elementwise_max(m[e], v);
        }
    }
    const u16x2_t a = __builtin_elementwise_max(__builtin_elementwise_max(m[0], m[1]), __builtin_elementwise_max(m[2], m[3]));
    return max(static_cast<uint32_t>(a.x), static_cast<uint32_t>(a.y));
}
// The value of such bits.
__device__ __forceinline__ float bf16_bits_value(uint32_t m) { return __uint_as_float(m << 16); }

// An OR over the workgroup's waves that does not wait for the loads in flight (__syncthreads_or
// would): each wave posts its vote into words[wave] here; after the next barrier that also waits
// for LDS (publish), or_votes reads the workgroup's OR.
__device__ __forceinline__ void post_vote(int* words, int wave, bool pred) {
    const bool any = __builtin_amdgcn_ballot_w64(pred) != 0;
    if ((threadIdx.x & 63) == 0) words[wave] = any ? 1 : 0;
}
__device__ __forceinline__ int or_votes(const int* words) {
    return __builtin_amdgcn_readfirstlane(words[0] | words[1] | words[2] | words[3]);
}

// Sum over the 8 lanes 8p' .. 8p' + 7 (an 8-lane group holds a row in the float32 tiles).
__device__ __forceinline__ float oct_sum(float v) {
    v += quad_f<0xB1>(v);                               // quad_perm [1, 0, 3, 2]
    v += quad_f<kXor2>(v);                              // quad_perm [2, 3, 0, 1]
    v += quad_f<0x141>(v);                              // row_half_mirror: the other quad of the 8
    return v;
}

// Largest of v over the same 8 lanes.
__device__ __forceinline__ float oct_max(float v) {
    v = fmaxf(v, quad_f<0xB1>(v));
    v = fmaxf(v, quad_f<kXor2>(v));
    v = fmaxf(v, quad_f<0x141>(v));
    return v;
}

// Dims 8e .. 8e + 7 of a bf16 row, rotated at position j (cos/sin from the table). Dim d pairs
// with d + 32 (e < 4: x' = x cos - y sin) or d - 32 (e >= 4: y' = y cos + x sin): dims of e ^ 4.
__device__ __forceinline__ void rot_eighth(const bf16_t* row, const float* cstab, int j, int e, float (&out)[8]) {
    const float sg = (e < 4) ? -1.f : 1.f;
    const uint4 ow = reinterpret_cast<const uint4*>(row)[e];
    const uint4 pw = reinterpret_cast<const uint4*>(row)[e ^ 4];
    const float4* cs = reinterpret_cast<const float4*>(cstab + static_cast<int64_t>(j) * 2 * kPairs + 16 * (e & 3));
    const uint32_t o4[4] = {ow.x, ow.y, ow.z, ow.w}, p4[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float4 t = cs[h];                          // (cos, sin) of dims 8e + 2h, + 1
        out[2 * h] = fmaf(sg * bf16_lo(p4[h]), t.y, bf16_lo(o4[h]) * t.x);
        out[2 * h + 1] = fmaf(sg * bf16_hi(p4[h]), t.w, bf16_hi(o4[h]) * t.z);
    }
}

// The range flag word (nonzero: flagged) of the staged rows that thread t of a tile checks: threads 0..3 the near block
// (rows i0 - 64 .. i0 + 63), thread 4 + 4n + u the u-th flag block of kept rung n's rows
// i0 - a - 1 .. i0 + 63 - a (clipped at 0), for rungs the tile reaches (at most 16: the matrix-core
// kernels' limit); every other thread none. The rung's floor comes from the uniform offset table by
// a per-lane choice among scalars: a per-lane index into the kernel arguments would be a vector
// load followed by a full wait behind every load in flight (here: the q burst).
template <typename Args>
__device__ __forceinline__ uint32_t rows_flagged(const Args& A, int grp, int i0, int n_reach) {
    const int t = threadIdx.x;
    int blk = -1;
    if (t < 4) {
        blk = i0 / kFlagRows - 2 + t;
    } else if (t < 4 + 4 * 16) {
        const int n = (t - 4) >> 2, u = (t - 4) & 3;
        if (n < n_reach) {
            int a = 0;
#pragma unroll
            for (int m = 0; m < 16; ++m) a = (n == m) ? A.off[m].a : a;
            const int lo = max(i0 - a - 1, 0), hi = min(i0 + kTile - 1 - a, A.L - 1);
            if (lo / kFlagRows + u <= hi / kFlagRows) blk = lo / kFlagRows + u;
        }
    }
    // every lane loads (word 0 where it checks none), so that the test of the word can wait until
    // the caller needs it instead of stalling the loads issued after this one
    const bool real = blk >= 0 && blk < A.n_blk;
    const uint32_t w = A.kvflags[real ? static_cast<int64_t>(grp) * A.n_blk + blk : 0];
    return real ? w : 0u;
}

}  // namespace mx
}  // namespace fibattn
