// Single-token decode of Fibonacci-offset sparse attention on gfx950: each sequence's new query
// attends, in the cache of its keys and values, to the window and the offset rungs of its own
// position.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention" (arXiv
// 2606.28560), §2 "Attended set" (window distances 0..W, one slot per rung at d = alpha f read by
// linear interpolation between rows pos - floor(d) and pos - floor(d) - 1, RoPE at true positions
// before the gather) and §2 "Implementation note" (integer offsets read one row). The result is
// the forward pass's output row at that position.
//
// A workgroup owns (batch b, key-value head g, 4 query heads): the rows its slots read are at
// most W + 1 window rows and two rows per kept rung, staged once in LDS as float32 (keys rotated
// at their own positions) and shared by the 4 query heads (GQA). Wave w then takes query head
// w: one slot per lane for the scores, a wave-wide softmax, one dim per lane for P.V. The work is
// a few thousand multiply-adds per head; the time is the latency of one round of row loads.
#include "fibattn_device.h"

namespace fibattn {

namespace {

constexpr int kRowsMax = kMaxWin + 2 * kMaxOff;         // window rows (W + 1 <= 32), then near / far of each rung
constexpr int kPitch = kD + 1;                           // LDS row pitch in floats (lanes reading
                                                         // different rows at one dim: distinct banks)
constexpr int kDecNT = 256;

template <typename T>
__global__ __launch_bounds__(kDecNT) void decode_kernel(DecodeArgs A) {
    constexpr float kNegInf = -__builtin_huge_valf();
    __shared__ float krows[kRowsMax * kPitch];
    __shared__ float vrows[kRowsMax * kPitch];
    __shared__ float qrot[4][kD];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n_chunk = (A.G + 3) >> 2;
    const int bg = blockIdx.x / n_chunk;                 // b * Hkv + g
    const int chunk = blockIdx.x % n_chunk;
    const int b = bg / A.Hkv, g = bg % A.Hkv;
    const int pos = A.pos[b];
    const bool pos_ok = pos >= 0 && pos < A.Lmax;
    const int W = A.W;
    const int n_rows = W + 1 + 2 * A.n_off;

    // ---- stage the rows: row r < W + 1 is distance r; row W + 1 + 2n (+1) is rung n's near (far)
    // row. Thread (row, c) takes dims 4c..4c+3 and 32 + 4c..: whole RoPE pairs. Rows before 0 (or
    // every row, for a position outside the cache) are zeros and are never used. ----
    const T* kc = static_cast<const T*>(A.kc) + static_cast<int64_t>(bg) * A.Lmax * kD;
    const T* vc = static_cast<const T*>(A.vc) + static_cast<int64_t>(bg) * A.Lmax * kD;
    for (int e = threadIdx.x; e < n_rows * 8; e += kDecNT) {
        const int r = e >> 3, c = e & 7;
        int dist;
        if (r <= W) {
            dist = r;
        } else {
            const int n = (r - W - 1) >> 1;
            dist = A.off[n].a + ((r - W - 1) & 1);
        }
        const int j = pos - dist;
        float4 k0 = make_float4(0.f, 0.f, 0.f, 0.f), k1 = k0, v0 = k0, v1 = k0;
        if (pos_ok && j >= 0) {
            k0 = load4<T>(kc + static_cast<int64_t>(j) * kD + 4 * c);
            k1 = load4<T>(kc + static_cast<int64_t>(j) * kD + kPairs + 4 * c);
            v0 = load4<T>(vc + static_cast<int64_t>(j) * kD + 4 * c);
            v1 = load4<T>(vc + static_cast<int64_t>(j) * kD + kPairs + 4 * c);
            const float x[4] = {k0.x, k0.y, k0.z, k0.w}, y[4] = {k1.x, k1.y, k1.z, k1.w};
            float rx[4], ry[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float cs, sn;
                rope_cos_sin(j, A.fr.hi[4 * c + u], A.fr.lo[4 * c + u], cs, sn);
                rx[u] = x[u] * cs - y[u] * sn;
                ry[u] = y[u] * cs + x[u] * sn;
            }
            k0 = make_float4(rx[0], rx[1], rx[2], rx[3]);
            k1 = make_float4(ry[0], ry[1], ry[2], ry[3]);
        }
        float* kr = krows + r * kPitch;
        float* vr = vrows + r * kPitch;
        kr[4 * c] = k0.x; kr[4 * c + 1] = k0.y; kr[4 * c + 2] = k0.z; kr[4 * c + 3] = k0.w;
        kr[kPairs + 4 * c] = k1.x; kr[kPairs + 4 * c + 1] = k1.y; kr[kPairs + 4 * c + 2] = k1.z; kr[kPairs + 4 * c + 3] = k1.w;
        vr[4 * c] = v0.x; vr[4 * c + 1] = v0.y; vr[4 * c + 2] = v0.z; vr[4 * c + 3] = v0.w;
        vr[kPairs + 4 * c] = v1.x; vr[kPairs + 4 * c + 1] = v1.y; vr[kPairs + 4 * c + 2] = v1.z; vr[kPairs + 4 * c + 3] = v1.w;
    }

    // ---- wave w: query head h, rotated at pos (lane j < 32 rotates pair j) ----
    const int hh = chunk * 4 + wave;                     // query head within the group
    const bool head_ok = hh < A.G;
    const int h = g * A.G + (head_ok ? hh : 0);
    const int64_t qrow = (static_cast<int64_t>(b) * A.Hq + h) * kD;
    {
        const float x = head_ok ? load_elem<T>(static_cast<const T*>(A.q) + qrow + lane) : 0.f;
        const float y = __shfl_xor(x, 32, 64);           // the other half of the pair
        float cs = 1.f, sn = 0.f;
        if (pos_ok) rope_cos_sin(pos, A.fr.hi[lane & 31], A.fr.lo[lane & 31], cs, sn);
        // lane j < 32: x_j cos - x_{j+32} sin; lane j >= 32: x_j cos + x_{j-32} sin
        qrot[wave][lane] = (lane < kPairs) ? x * cs - y * sn : x * cs + y * sn;
    }
    __syncthreads();

    // ---- scores: lane s is slot s (window distance s <= W, then rung s - W - 1) ----
    const int n_slots = W + 1 + A.n_off;
    float sc = kNegInf;
    if (lane < n_slots && pos_ok) {
        int rn, rf = -1;
        float t = 0.f;
        bool valid;
        if (lane <= W) {
            rn = lane;
            valid = pos >= lane;
        } else {
            const int n = lane - W - 1;
            rn = W + 1 + 2 * n;
            if (A.off[n].interp) {
                rf = rn + 1;
                t = A.off[n].t;
            }
            valid = pos >= A.off[n].a + A.off[n].interp;
        }
        if (valid) {
            const float* kn = krows + rn * kPitch;
            float dn = 0.f, df = 0.f;
#pragma unroll 16
            for (int d = 0; d < kD; ++d) dn = fmaf(qrot[wave][d], kn[d], dn);
            if (rf >= 0) {
                const float* kf = krows + rf * kPitch;
#pragma unroll 16
                for (int d = 0; d < kD; ++d) df = fmaf(qrot[wave][d], kf[d], df);
            }
            sc = fmaf(t, df - dn, dn) * A.scale;
        }
    }
    float m = sc;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float p = (sc == kNegInf) ? 0.f : expf(sc - m);
    float l = p;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);

    // ---- P.V: lane d is dim d; the slots in order, each blended like its key ----
    float acc = 0.f;
    for (int s = 0; s < n_slots; ++s) {
        const float ps = __shfl(p, s, 64);
        if (s <= W) {
            acc = fmaf(ps, vrows[s * kPitch + lane], acc);
        } else {
            const int n = s - W - 1;
            const int rn = W + 1 + 2 * n;
            const float t = A.off[n].interp ? A.off[n].t : 0.f;
            const float vn = vrows[rn * kPitch + lane], vf = vrows[(rn + 1) * kPitch + lane];
            acc = fmaf(ps, fmaf(t, vf - vn, vn), acc);
        }
    }
    if (head_ok) {
        const float nan = __builtin_nanf("");
        const float out = pos_ok ? acc / l : nan;
        store_elem<T>(static_cast<T*>(A.o) + qrow + lane, out);
        if (A.lse != nullptr && lane == 0)
            A.lse[static_cast<int64_t>(b) * A.Hq + h] = pos_ok ? m + logf(l) : nan;
    }
}

}  // namespace

hipError_t launch_decode(int dtype, const DecodeArgs& A, hipStream_t s) {
    const unsigned blocks = static_cast<unsigned>(A.B * A.Hkv * ((A.G + 3) / 4));
    if (dtype == 0)
        hipLaunchKernelGGL(decode_kernel<float>, dim3(blocks), dim3(kDecNT), 0, s, A);
    else
        hipLaunchKernelGGL(decode_kernel<bf16_t>, dim3(blocks), dim3(kDecNT), 0, s, A);
    return hipGetLastError();
}

}  // namespace fibattn
