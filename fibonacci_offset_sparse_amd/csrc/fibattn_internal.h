// Internal declarations shared by the host library and the gfx950 kernels of libfibattn.so.
// Nothing here is part of the C ABI (include/fibattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fibattn {

constexpr int kD = 64;        // head dimension the kernels take
constexpr int kPairs = 32;    // RoPE pairs (j, j + 32)
constexpr int kTile = 64;     // query (or key) positions per workgroup
constexpr int kMaxWin = 32;   // window slots 0..W with W <= 31
constexpr int kMaxOff = 32;   // base rungs
// backward stages (the bit values of the public stage mask)
constexpr int kStagePrep = 1, kStageQuery = 2, kStageKey = 4;

// Range flags of the staged rows: one word per (group of kPrepRowGroup consecutive (batch, head)
// rows, block of kFlagRows positions), byte w of it for positions 8w .. 8w + 7 of the block.
constexpr int kPrepRowGroup = 4;
constexpr int kFlagRows = 32;

// One kept offset of the plan (DUP rungs are removed before launch).
struct OffsetSlot {
    int32_t a;       // distance of the nearer row, floor(d)
    float t;         // weight of the farther row a + 1 (0 for an integral offset)
    int32_t interp;  // 1: interpolated, valid for i >= a + 1; 0: integral, valid for i >= a
    int32_t f;       // base rung (d(alpha) weight)
};

// The first 16 kept rungs' floors and reach, packed for the matrix-core kernels' scans of the rungs
// a tile reaches (a few wide scalar loads instead of one load of the offset table per rung). Both
// are non-decreasing in the rung (the distances alpha f increase), so a count of entries under a
// bound is the length of the prefix under it; entries past the kept rungs hold kScanPast.
constexpr int kScanRungs = 16;
constexpr int32_t kScanPast = 1 << 30;
struct RungScan {
    int32_t a[kScanRungs];   // floor(d) of kept rung n
    int32_t r[kScanRungs];   // a + 1 for an interpolated rung, a for an integral one: its first query
};

// RoPE frequencies omega_j / (2 pi) as an unevaluated float sum hi + lo (double accuracy).
struct RopeFreq {
    float hi[kPairs];
    float lo[kPairs];
};

struct RopeKeysArgs {
    const void* k;   // [B*Hkv, L, 64] storage type
    float* krot;     // [B*Hkv, L, 64] float32
    int32_t n_bh;    // B * Hkv
    int32_t L;
    RopeFreq fr;
};

// bf16 storage: rotated keys and values as fp16 rows for the matrix-core forward and backward
// (one layout for both: element 4m + c of a row holds dim 16c + m).
struct PrepArgs {
    const void* k;       // [B*Hkv, L, 64] bf16
    const void* v;       // [B*Hkv, L, 64] bf16
    _Float16* k16;       // [B*Hkv, L, 64] rotated keys, dims permuted
    _Float16* v16;       // [B*Hkv, L, 64] values, dims permuted
    float* cs;           // [L, 32, 2] cos and sin of every position and RoPE pair
    // the low parts of the rotated keys, krot - fp16(krot) as fp16 (same layout as k16), or
    // nullptr; with main == 0 only these are written (k16, v16 and cs are left alone)
    _Float16* k16lo;
    int32_t main;
    // per (group of kPrepRowGroup (batch, head) rows, block of 32 positions): nonzero when a key or
    // value row of the block lies outside the range fp16 holds exactly enough (written when main)
    uint32_t* flags;
    int32_t n_blk;       // ceil(L / 32)
    int32_t n_bh;
    int32_t L;
    RopeFreq fr;
};

struct FwdArgs {
    const void* q;       // [B, Hq, L, 64] storage type
    const void* kstage;  // [B, Hkv, L, 64] rotated keys: float32 in dim order (f32 storage) or fp16
                         // with dims permuted, element 4m + c holding dim 16c + m (bf16 storage)
    const void* vstage;  // [B, Hkv, L, 64] values: the input (f32 storage) or fp16, dims permuted
    const void* v;       // [B, Hkv, L, 64] the caller's values
    const void* k;       // [B, Hkv, L, 64] the caller's keys (unrotated)
    const float* cstab;  // [L, 32, 2] cos/sin table (bf16 storage)
    const uint32_t* kvflags;  // range flags of the staged rows (bf16 storage), see PrepArgs
    int32_t n_blk;
    void* o;             // [B, Hq, L, 64]
    float* lse;          // [B, Hq, L] or nullptr
    int32_t B, L, Hq, Hkv, G, W, n_off;
    int32_t xcd_map;     // matrix-core kernels: 0 plain order, 1 each (batch, kv head) on one XCD, 2 also mix tiles per CU,
                         // 3 each unit on one XCD, groups of four units tile-major
    float qscale;        // log2(e) / sqrt(D): scores kept in base 2
    RopeFreq fr;
    OffsetSlot off[kMaxOff];
    RungScan scan;
};

struct BwdArgs {
    const void* q;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    const float* krot;   // [B, Hkv, L, 64] float32 (workspace)
    float* qrot;         // [B, Hq, L, 64] float32 (workspace)
    float* pbuf;         // [B, Hq, S, L] softmax weights (workspace)
    float* dsbuf;        // [B, Hq, S, L] score gradients, already times 1/sqrt(D) (workspace)
    float* partial;      // [n_wg, kMaxOff] per-workgroup sums of d(loss)/dt (workspace)
    void* dq;
    void* dk;
    void* dv;
    float* dalpha;
    float* dtheta;
    int32_t B, L, Hq, Hkv, G, W, n_off, S;
    int32_t n_wg;        // workgroups of the query-centric kernel
    float scale;         // 1/sqrt(D)
    float dalpha_dtheta;
    RopeFreq fr;
    OffsetSlot off[kMaxOff];
    RungScan scan;
    // matrix-core path (bfloat16 storage): staged rows from prep_kv16 (the forward's own), and
    // what the query-side kernel hands the key-side kernel; rows with dims permuted have element
    // 4m + c holding dim 16c + m
    const void* kstage;  // [B*Hkv, L, 64] fp16 rotated keys, dims permuted
    const void* vstage;  // [B*Hkv, L, 64] fp16 values, dims permuted
    const float* cstab;  // [L, 32, 2] cos, sin
    const uint32_t* kvflags;  // range flags of the staged rows, see PrepArgs
    int32_t n_blk;
    const void* k;       // [B, Hkv, L, 64] the caller's keys (unrotated)
    const void* kstage_lo;  // [B*Hkv, L, 64] fp16 low parts of the rotated keys (precise scores)
    void* qrot16;        // [B, Hq, L, 64] fp16 rotated queries, dims permuted
    void* do16;          // [B, Hq, L, 64] fp16 copy of dout, dims permuted
    // per query and head, fp16 pairs (p low, dS/sqrt(D) high): the window distances 0..15 of each
    // query ([B, Hq, L, kNW]), and each rung's entry without its coefficients, rung-major
    // ([B, Hq, kNR, L])
    uint32_t* wwin;
    uint32_t* wrung;
    // per (batch, head, query tile): the powers of two the query side scaled that tile's hand-off
    // by (q, do, dS; bytes of one word)
    uint32_t* exps;
    // [0]: the call number of the last query stage run over this workspace; [1]: that of the last
    // query stage that left some tile to the float32 kernel; [2]: that of the last query stage
    // with some tile's exponents not all 0 (written by the query kernel)
    uint64_t* seqw;
    uint64_t seq;        // this call's number (the host's count of backward calls, from 1)
    int32_t q_fp32_wg;   // workgroups of this call's query stage (0 without it): its float32 tiles
    int32_t q_xcd_map;   // the query kernel's tile order
    float qscale;        // log2(e)/sqrt(D)
    int32_t xcd_map;
};

// Single-token decode: each sequence's new query against its cache.
struct DecodeArgs {
    const void* q;       // [B, Hq, 64] storage type: the new query of each sequence
    const void* kc;      // [B, Hkv, Lmax, 64] storage type: unrotated keys, rows 0..pos[b] valid
    const void* vc;      // [B, Hkv, Lmax, 64] storage type
    const int32_t* pos;  // [B] device: the position of each sequence's new token
    void* o;             // [B, Hq, 64]
    float* lse;          // [B, Hq] or nullptr
    int32_t B, Lmax, Hq, Hkv, G, W, n_off;
    float scale;         // 1/sqrt(D)
    RopeFreq fr;
    OffsetSlot off[kMaxOff];
};

// Entries per query in the weight tables of the matrix-core backward: 16 window distances, 16 rungs.
constexpr int kNW = 16, kNR = 16;

// Sets the calling thread's error text (fibattn_last_error) and returns status (an int of
// fibattn_status_t).
int report_error(int status, const char* fmt, ...);

hipError_t launch_rope_keys(int dtype, const RopeKeysArgs& a, hipStream_t s);
// keys and values with dims permuted (element 4m + c of a row holds dim 16c + m), and the table
hipError_t launch_prep_kv16(const PrepArgs& a, hipStream_t s);
hipError_t launch_fwd_attend(int dtype, const FwdArgs& a, hipStream_t s);
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s);
bool fwd_mfma_supported(const FwdArgs& a);
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd(int dtype, const BwdArgs& a, bool want_dalpha, int stages, hipStream_t s);
bool bwd_mfma_supported(const BwdArgs& a);
hipError_t launch_bwd_mfma(const BwdArgs& a, bool want_dalpha, int stages, hipStream_t s);
hipError_t launch_dalpha(const BwdArgs& a, hipStream_t s);
int bwd_query_workgroups(int B, int L, int Hkv, int G);

}  // namespace fibattn
