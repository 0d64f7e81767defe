// Host side of libfibattn.so: argument checks, the offset plan, schedules, workspace layout and
// kernel dispatch behind the C ABI of include/fibattn.h.
//
// Section references are to "Depth-Staggered Fibonacci Spacing for Sparse Attention: Static
// Schedules Beat Learned Dilation and Extrapolate Where Dense Attention Fails" (arXiv 2606.28560).
#include "fibattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fibattn_internal.h"

using namespace fibattn;

namespace {

thread_local char g_error[512] = "";

fibattn_status_t fail(fibattn_status_t status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return status;
}

fibattn_status_t hip_fail(hipError_t e, const char* what) {
    return fail(FIBATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// §2 "Attended set": the base sequence, K = 15.
constexpr int32_t kFib[15] = {1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987};
// §2 "Per-layer scalar": the coprime stride.
constexpr int32_t kCoprimeStride = 7;
// Absolute tolerance under which alpha * f counts as integral.
constexpr double kSnapTol = 1e-9;
constexpr int32_t kMaxL = 1 << 20;

struct Plan {
    int n_keep = 0;          // kept offsets (INT and INTERP)
    bool any_integral = false;
    OffsetSlot keep[kMaxOff] = {};
};

// The scan table of a plan's first kScanRungs kept rungs (RungScan).
RungScan rung_scan(const Plan& plan) {
    RungScan sc;
    for (int n = 0; n < kScanRungs; ++n) {
        const bool kept = n < plan.n_keep;
        sc.a[n] = kept ? plan.keep[n].a : kScanPast;
        sc.r[n] = kept ? plan.keep[n].a + plan.keep[n].interp : kScanPast;
    }
    return sc;
}

fibattn_status_t check_offsets(double alpha, int32_t W, const int32_t* offsets, int32_t K) {
    if (K < 0 || K > FIBATTN_MAX_K) return fail(FIBATTN_ERR_INVALID, "K = %d outside [0, %d]", K, FIBATTN_MAX_K);
    if (K > 0 && offsets == nullptr) return fail(FIBATTN_ERR_INVALID, "offsets is NULL");
    if (W < 0) return fail(FIBATTN_ERR_INVALID, "W = %d < 0", W);
    if (!std::isfinite(alpha) || alpha <= 0.0) return fail(FIBATTN_ERR_INVALID, "alpha = %g is not finite and > 0", alpha);
    for (int32_t k = 0; k < K; ++k) {
        if (offsets[k] < 1) return fail(FIBATTN_ERR_INVALID, "offsets[%d] = %d < 1", k, offsets[k]);
        if (k > 0 && offsets[k] <= offsets[k - 1])
            return fail(FIBATTN_ERR_INVALID, "offsets not strictly increasing at %d", k);
        if (alpha * static_cast<double>(offsets[k]) > static_cast<double>(1 << 30))
            return fail(FIBATTN_ERR_UNSUPPORTED, "alpha * offsets[%d] exceeds 2^30", k);
    }
    return FIBATTN_OK;
}

// One rung: d = alpha f in double, snapped to the nearest integer within kSnapTol.
void plan_one(double alpha, int32_t W, int32_t f, uint8_t& kind, int32_t& a, double& t, int32_t& reach) {
    double d = alpha * static_cast<double>(f);
    const double r = std::nearbyint(d);
    if (std::fabs(d - r) <= kSnapTol) d = r;
    const double fl = std::floor(d);
    a = static_cast<int32_t>(fl);
    if (d == fl) {
        kind = (a <= W) ? FIBATTN_DUP : FIBATTN_INT;
        t = 0.0;
        reach = a;
    } else {
        kind = FIBATTN_INTERP;
        t = d - fl;
        reach = a + 1;
    }
}

Plan make_plan(double alpha, int32_t W, const int32_t* offsets, int32_t K) {
    Plan p;
    for (int32_t k = 0; k < K; ++k) {
        uint8_t kind;
        int32_t a, reach;
        double t;
        plan_one(alpha, W, offsets[k], kind, a, t, reach);
        if (kind != FIBATTN_INTERP) p.any_integral = true;
        if (kind == FIBATTN_DUP) continue;
        OffsetSlot& s = p.keep[p.n_keep++];
        s.a = a;
        s.t = static_cast<float>(t);
        s.interp = (kind == FIBATTN_INTERP) ? 1 : 0;
        s.f = offsets[k];
    }
    return p;
}

// Scores are kept in base 2: q.k * log2(e) / sqrt(D).
float score_scale() { return static_cast<float>(1.4426950408889634074 / std::sqrt(static_cast<double>(kD))); }

RopeFreq make_freq(double theta) {
    RopeFreq fr;
    for (int j = 0; j < kPairs; ++j) {
        const double omega = std::pow(theta, -2.0 * j / kD);
        const double c = omega / (2.0 * M_PI);
        fr.hi[j] = static_cast<float>(c);
        fr.lo[j] = static_cast<float>(c - static_cast<double>(fr.hi[j]));
    }
    return fr;
}

fibattn_status_t check_dims(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t W,
                            int32_t dtype, double rope_theta) {
    if (B < 1 || L < 1 || Hq < 1 || Hkv < 1)
        return fail(FIBATTN_ERR_INVALID, "B, L, Hq, Hkv must be >= 1 (got %d, %d, %d, %d)", B, L, Hq, Hkv);
    if (Hq % Hkv != 0) return fail(FIBATTN_ERR_INVALID, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
    if (dtype != FIBATTN_F32 && dtype != FIBATTN_BF16) return fail(FIBATTN_ERR_INVALID, "unknown dtype %d", dtype);
    if (!std::isfinite(rope_theta) || rope_theta <= 0.0)
        return fail(FIBATTN_ERR_INVALID, "rope_theta = %g is not finite and > 0", rope_theta);
    if (W < 0) return fail(FIBATTN_ERR_INVALID, "W = %d < 0", W);
    if (D != kD) return fail(FIBATTN_ERR_UNSUPPORTED, "head dim D = %d (only 64 is implemented)", D);
    if (W > FIBATTN_MAX_W) return fail(FIBATTN_ERR_UNSUPPORTED, "W = %d > %d", W, FIBATTN_MAX_W);
    if (L > kMaxL) return fail(FIBATTN_ERR_UNSUPPORTED, "L = %d > %d", L, kMaxL);
    if (B > 65535 || Hq > 65535) return fail(FIBATTN_ERR_UNSUPPORTED, "B or Hq above 65535");
    if (static_cast<int64_t>(B) * Hkv > 4 * 65535)
        return fail(FIBATTN_ERR_UNSUPPORTED, "B * Hkv above %d", 4 * 65535);
    return FIBATTN_OK;
}

size_t elem_bytes(int32_t dtype) { return dtype == FIBATTN_F32 ? 4 : 2; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Staged keys (and values) of the forward: float32 rotated keys for float32 storage, or fp16
// rotated keys followed by fp16 values for bf16 storage; the same bytes either way.
size_t krot_bytes(int32_t B, int32_t L, int32_t Hkv) {
    return align256(static_cast<size_t>(B) * Hkv * L * kD * sizeof(float));
}
size_t half_rows_bytes(int32_t B, int32_t L, int32_t Hkv) {
    return static_cast<size_t>(B) * Hkv * L * kD * sizeof(uint16_t);
}
// cos/sin table [L, 32, 2] float32 after the staged rows (bf16 storage)
size_t cs_table_bytes(int32_t L) { return align256(static_cast<size_t>(L) * kPairs * 2 * sizeof(float)); }
int32_t flag_blocks(int32_t L) { return (L + kFlagRows - 1) / kFlagRows; }
// range flags of the staged rows (bf16 storage): one word per (group of kPrepRowGroup (batch, head)
// rows, block of kFlagRows positions), after the table
size_t flags_bytes(int32_t B, int32_t L, int32_t Hkv) {
    const size_t groups = (static_cast<size_t>(B) * Hkv + kPrepRowGroup - 1) / kPrepRowGroup;
    return align256(groups * flag_blocks(L) * sizeof(uint32_t));
}
size_t fwd_ws_bytes(int32_t B, int32_t L, int32_t Hkv) {
    return krot_bytes(B, L, Hkv) + cs_table_bytes(L) + flags_bytes(B, L, Hkv);
}
uint32_t* flags_at(void* ws, int32_t B, int32_t L, int32_t Hkv) {
    return reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + krot_bytes(B, L, Hkv) + cs_table_bytes(L));
}

// Workspace of the matrix-core backward (bfloat16 storage): staged fp16 keys and values and the
// cos/sin table (the forward's layout of the same sizes), the rotated queries (fp16), the per key
// row term weights, and the per-workgroup d(loss)/dt partials.
struct BwdFastLayout {
    size_t qrot, do16, wwin, wrung, part, klo, exps, seqw, total;
};
BwdFastLayout bwd_fast_layout(int32_t B, int32_t L, int32_t Hq, int32_t Hkv) {
    BwdFastLayout f;
    f.qrot = fwd_ws_bytes(B, L, Hkv);
    f.do16 = f.qrot + align256(static_cast<size_t>(B) * Hq * L * kD * sizeof(uint16_t));
    f.wwin = f.do16 + align256(static_cast<size_t>(B) * Hq * L * kD * sizeof(uint16_t));
    f.wrung = f.wwin + align256(static_cast<size_t>(B) * Hq * L * kNW * sizeof(uint32_t));
    f.part = f.wrung + align256(static_cast<size_t>(B) * Hq * L * kNR * sizeof(uint32_t));
    const size_t n_wg = static_cast<size_t>(bwd_query_workgroups(B, L, Hkv, Hq / Hkv));
    f.klo = f.part + align256(n_wg * kMaxOff * sizeof(float));
    // low parts of the rotated keys (fp16), for the precise scores of a call that asks for d(alpha)
    f.exps = f.klo + align256(half_rows_bytes(B, L, Hkv));
    // the query tiles' scale exponents [B, Hq, tiles]
    f.seqw = f.exps + align256(static_cast<size_t>(B) * Hq * ((L + kTile - 1) / kTile) * sizeof(uint32_t));
    // two call numbers: the last query stage run over this workspace, the last one with float32 tiles
    f.total = f.seqw + 256;
    return f;
}

}  // namespace

int fibattn::report_error(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return status;
}

namespace {

#define FIBATTN_TRY(expr)                        \
    do {                                         \
        const fibattn_status_t st_ = (expr);     \
        if (st_ != FIBATTN_OK) return st_;       \
    } while (0)

}  // namespace

extern "C" {

const char* fibattn_status_string(fibattn_status_t s) {
    switch (s) {
        case FIBATTN_OK: return "ok";
        case FIBATTN_ERR_INVALID: return "invalid argument";
        case FIBATTN_ERR_UNSUPPORTED: return "unsupported argument";
        case FIBATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case FIBATTN_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char* fibattn_last_error(void) { return g_error; }

fibattn_status_t fibattn_base_offsets(int32_t base, int32_t pow2_max, int32_t* out, int32_t capacity,
                                      int32_t* count) {
    g_error[0] = '\0';
    if (out == nullptr || count == nullptr) return fail(FIBATTN_ERR_INVALID, "NULL output");
    int32_t n = 0;
    int32_t tmp[FIBATTN_MAX_K];
    if (base == FIBATTN_BASE_FIB) {
        for (int32_t f : kFib) tmp[n++] = f;
    } else if (base == FIBATTN_BASE_POW2) {
        if (pow2_max < 1) return fail(FIBATTN_ERR_INVALID, "pow2_max = %d < 1", pow2_max);
        for (int64_t f = 1; f <= pow2_max && n < FIBATTN_MAX_K; f <<= 1) tmp[n++] = static_cast<int32_t>(f);
    } else {
        return fail(FIBATTN_ERR_INVALID, "unknown base %d", base);
    }
    if (capacity < n) return fail(FIBATTN_ERR_INVALID, "capacity %d < %d rungs", capacity, n);
    std::memcpy(out, tmp, sizeof(int32_t) * n);
    *count = n;
    return FIBATTN_OK;
}

fibattn_status_t fibattn_round_offsets(double alpha, const int32_t* offsets, int32_t K, int32_t* out,
                                       int32_t capacity, int32_t* count) {
    g_error[0] = '\0';
    if (out == nullptr || count == nullptr) return fail(FIBATTN_ERR_INVALID, "NULL output");
    FIBATTN_TRY(check_offsets(alpha, 0, offsets, K));
    // d = alpha f with 2d snapped to an integer within kSnapTol (an exact integer or half-integer
    // distance), then rounded to the nearest integer, ties to even (nearbyint in the default
    // rounding mode); rungs are increasing, so equal distances are adjacent
    int32_t tmp[FIBATTN_MAX_K];
    int32_t n = 0;
    for (int32_t k = 0; k < K; ++k) {
        double d2 = 2.0 * alpha * static_cast<double>(offsets[k]);
        const double r2 = std::nearbyint(d2);
        if (std::fabs(d2 - r2) <= kSnapTol) d2 = r2;
        const int32_t d = static_cast<int32_t>(std::nearbyint(0.5 * d2));
        if (d < 1 || (n > 0 && d == tmp[n - 1])) continue;
        tmp[n++] = d;
    }
    if (capacity < n) return fail(FIBATTN_ERR_INVALID, "capacity %d < %d distances", capacity, n);
    if (n > 0) std::memcpy(out, tmp, sizeof(int32_t) * n);
    *count = n;
    return FIBATTN_OK;
}

fibattn_status_t fibattn_alpha_schedule(int32_t schedule, int32_t layer, int32_t n_layers, double* alpha) {
    g_error[0] = '\0';
    if (alpha == nullptr) return fail(FIBATTN_ERR_INVALID, "NULL alpha");
    if (n_layers < 2) return fail(FIBATTN_ERR_INVALID, "n_layers = %d < 2", n_layers);
    if (layer < 0 || layer >= n_layers) return fail(FIBATTN_ERR_INVALID, "layer %d outside [0, %d)", layer, n_layers);
    switch (schedule) {
        case FIBATTN_SCHEDULE_FIXED: *alpha = 1.0; return FIBATTN_OK;
        case FIBATTN_SCHEDULE_LINEAR:
            *alpha = 0.5 + static_cast<double>(layer) / static_cast<double>(n_layers - 1);
            return FIBATTN_OK;
        case FIBATTN_SCHEDULE_COPRIME: {
            int32_t a = kCoprimeStride, b = n_layers;
            while (b != 0) { const int32_t r = a % b; a = b; b = r; }
            if (a != 1) return fail(FIBATTN_ERR_INVALID, "n_layers = %d shares a factor with 7", n_layers);
            const int32_t m = static_cast<int32_t>((static_cast<int64_t>(kCoprimeStride) * layer) % n_layers);
            *alpha = 0.5 + static_cast<double>(m) / static_cast<double>(n_layers - 1);
            return FIBATTN_OK;
        }
    }
    return fail(FIBATTN_ERR_INVALID, "unknown schedule %d", schedule);
}

fibattn_status_t fibattn_alpha_from_theta(double theta, double* alpha, double* dalpha_dtheta) {
    g_error[0] = '\0';
    if (!std::isfinite(theta)) return fail(FIBATTN_ERR_INVALID, "theta is not finite");
    const double s = 1.0 / (1.0 + std::exp(-theta));
    if (alpha != nullptr) *alpha = 0.5 + s;
    if (dalpha_dtheta != nullptr) *dalpha_dtheta = s * (1.0 - s);
    return FIBATTN_OK;
}

fibattn_status_t fibattn_plan(double alpha, int32_t W, const int32_t* offsets, int32_t K, uint8_t* kind_out,
                              int32_t* floor_out, float* t_out, int32_t* reach_out) {
    g_error[0] = '\0';
    FIBATTN_TRY(check_offsets(alpha, W, offsets, K));
    if (K > 0 && (kind_out == nullptr || floor_out == nullptr || t_out == nullptr || reach_out == nullptr))
        return fail(FIBATTN_ERR_INVALID, "NULL output array");
    for (int32_t k = 0; k < K; ++k) {
        double t;
        plan_one(alpha, W, offsets[k], kind_out[k], floor_out[k], t, reach_out[k]);
        t_out[k] = static_cast<float>(t);
    }
    return FIBATTN_OK;
}

size_t fibattn_fwd_workspace_bytes(int32_t B, int32_t L, int32_t Hkv, int32_t D, int32_t dtype) {
    (void)D;
    (void)dtype;
    if (B < 1 || L < 1 || Hkv < 1) return 0;
    return fwd_ws_bytes(B, L, Hkv);
}

fibattn_status_t fibattn_fwd_prep(const void* k, const void* v, int32_t B, int32_t L, int32_t Hkv, int32_t D,
                                  int32_t dtype, double rope_theta, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    g_error[0] = '\0';
    FIBATTN_TRY(check_dims(B, L, Hkv, Hkv, D, 0, dtype, rope_theta));
    if (k == nullptr || v == nullptr) return fail(FIBATTN_ERR_INVALID, "k or v is NULL");
    const size_t need = fwd_ws_bytes(B, L, Hkv);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FIBATTN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    hipError_t e;
    if (dtype == FIBATTN_F32) {
        RopeKeysArgs a;
        a.k = k;
        a.krot = static_cast<float*>(workspace);
        a.n_bh = B * Hkv;
        a.L = L;
        a.fr = make_freq(rope_theta);
        e = launch_rope_keys(dtype, a, static_cast<hipStream_t>(stream));
    } else {
        PrepArgs a;
        a.k = k;
        a.v = v;
        a.k16 = static_cast<_Float16*>(workspace);
        a.v16 = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) + half_rows_bytes(B, L, Hkv));
        a.cs = reinterpret_cast<float*>(static_cast<char*>(workspace) + krot_bytes(B, L, Hkv));
        a.n_bh = B * Hkv;
        a.L = L;
        a.fr = make_freq(rope_theta);
        a.k16lo = nullptr;
        a.main = 1;
        a.flags = flags_at(workspace, B, L, Hkv);
        a.n_blk = flag_blocks(L);
        e = launch_prep_kv16(a, static_cast<hipStream_t>(stream));
    }
    if (e != hipSuccess) return hip_fail(e, "forward prep launch");
    return FIBATTN_OK;
}

fibattn_status_t fibattn_fwd_attend(const void* q, const void* k, const void* v, double alpha, int32_t W,
                                    const int32_t* offsets, int32_t K, int32_t B, int32_t L, int32_t Hq, int32_t Hkv,
                                    int32_t D, int32_t dtype, double rope_theta, void* o, float* lse,
                                    const void* workspace, size_t workspace_bytes, void* stream) {
    g_error[0] = '\0';
    FIBATTN_TRY(check_dims(B, L, Hq, Hkv, D, W, dtype, rope_theta));
    FIBATTN_TRY(check_offsets(alpha, W, offsets, K));
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(FIBATTN_ERR_INVALID, "q, k, v or o is NULL");
    const size_t need = fwd_ws_bytes(B, L, Hkv);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FIBATTN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    const Plan plan = make_plan(alpha, W, offsets, K);
    FwdArgs a{};
    a.q = q;
    a.kstage = workspace;
    a.vstage = dtype == FIBATTN_F32 ? v : static_cast<const char*>(workspace) + half_rows_bytes(B, L, Hkv);
    a.cstab = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + krot_bytes(B, L, Hkv));
    a.kvflags = flags_at(const_cast<void*>(workspace), B, L, Hkv);
    a.n_blk = flag_blocks(L);
    a.v = v;
    a.k = k;
    a.xcd_map = 0;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.L = L;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.W = W;
    a.n_off = plan.n_keep;
    a.qscale = score_scale();
    a.fr = make_freq(rope_theta);
    std::memcpy(a.off, plan.keep, sizeof(plan.keep));
    a.scan = rung_scan(plan);
    const hipError_t e = launch_fwd_attend(dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "fwd_attend launch");
    return FIBATTN_OK;
}

fibattn_status_t fibattn_fwd(const void* q, const void* k, const void* v, double alpha, int32_t W,
                             const int32_t* offsets, int32_t K, int32_t B, int32_t L, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t dtype, double rope_theta, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
    g_error[0] = '\0';
    // check everything before queueing the first kernel
    FIBATTN_TRY(check_dims(B, L, Hq, Hkv, D, W, dtype, rope_theta));
    FIBATTN_TRY(check_offsets(alpha, W, offsets, K));
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return fail(FIBATTN_ERR_INVALID, "q, k, v or o is NULL");
    FIBATTN_TRY(fibattn_fwd_prep(k, v, B, L, Hkv, D, dtype, rope_theta, workspace, workspace_bytes, stream));
    return fibattn_fwd_attend(q, k, v, alpha, W, offsets, K, B, L, Hq, Hkv, D, dtype, rope_theta, o, lse, workspace,
                              workspace_bytes, stream);
}

fibattn_status_t fibattn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* positions,
                                double alpha, int32_t W, const int32_t* offsets, int32_t K, int32_t B, int32_t Lmax,
                                int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype, double rope_theta, void* o,
                                float* lse, void* stream) {
    g_error[0] = '\0';
    FIBATTN_TRY(check_dims(B, Lmax, Hq, Hkv, D, W, dtype, rope_theta));
    FIBATTN_TRY(check_offsets(alpha, W, offsets, K));
    if (q == nullptr || k_cache == nullptr || v_cache == nullptr || positions == nullptr || o == nullptr)
        return fail(FIBATTN_ERR_INVALID, "q, k_cache, v_cache, positions or o is NULL");
    const Plan plan = make_plan(alpha, W, offsets, K);
    DecodeArgs a{};
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.pos = positions;
    a.o = o;
    a.lse = lse;
    a.B = B;
    a.Lmax = Lmax;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.W = W;
    a.n_off = plan.n_keep;
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(kD)));
    a.fr = make_freq(rope_theta);
    std::memcpy(a.off, plan.keep, sizeof(plan.keep));
    const hipError_t e = launch_decode(dtype, a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return FIBATTN_OK;
}

size_t fibattn_bwd_workspace_bytes(int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t W, int32_t K,
                                   int32_t dtype) {
    (void)D;
    (void)dtype;
    if (B < 1 || L < 1 || Hq < 1 || Hkv < 1 || W < 0 || K < 0 || Hq % Hkv != 0) return 0;
    const size_t S = static_cast<size_t>(W) + 1 + K;
    const size_t qrot = align256(static_cast<size_t>(B) * Hq * L * kD * sizeof(float));
    const size_t slots = align256(static_cast<size_t>(B) * Hq * S * L * sizeof(float));
    const size_t n_wg = static_cast<size_t>(bwd_query_workgroups(B, L, Hkv, Hq / Hkv));
    const size_t part = align256(n_wg * kMaxOff * sizeof(float));
    const size_t general = krot_bytes(B, L, Hkv) + qrot + 2 * slots + part;
    return std::max(general, bwd_fast_layout(B, L, Hq, Hkv).total);
}

int32_t fibattn_bwd_reuses_fwd_prep(double alpha, int32_t W, const int32_t* offsets, int32_t K, int32_t B,
                                    int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype) {
    g_error[0] = '\0';
    if (check_dims(B, L, Hq, Hkv, D, W, dtype, 1e4) != FIBATTN_OK) return 0;
    if (check_offsets(alpha, W, offsets, K) != FIBATTN_OK) return 0;
    if (dtype == FIBATTN_F32) return 1;   // both run rope_keys into the workspace's first array
    const Plan plan = make_plan(alpha, W, offsets, K);
    BwdArgs a{};
    a.G = Hq / Hkv;
    a.W = W;
    a.n_off = plan.n_keep;
    return bwd_mfma_supported(a) ? 1 : 0;   // else the backward rotates float32 keys of its own
}

fibattn_status_t fibattn_bwd_stages(int32_t stages, const void* q, const void* k, const void* v,
                                    const void* dout, double alpha, int32_t W, const int32_t* offsets, int32_t K,
                                    int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                                    double rope_theta, double dalpha_dtheta, void* dq, void* dk, void* dv,
                                    float* dalpha, float* dtheta, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    g_error[0] = '\0';
    if (stages < 1 || stages > FIBATTN_STAGE_ALL)
        return fail(FIBATTN_ERR_INVALID, "stage mask %d outside [1, %d]", stages, FIBATTN_STAGE_ALL);
    FIBATTN_TRY(check_dims(B, L, Hq, Hkv, D, W, dtype, rope_theta));
    FIBATTN_TRY(check_offsets(alpha, W, offsets, K));
    if (q == nullptr || k == nullptr || v == nullptr || dout == nullptr || dq == nullptr || dk == nullptr ||
        dv == nullptr)
        return fail(FIBATTN_ERR_INVALID, "a required pointer is NULL");
    if (!std::isfinite(dalpha_dtheta)) return fail(FIBATTN_ERR_INVALID, "dalpha_dtheta is not finite");
    const size_t need = fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, W, K, dtype);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(FIBATTN_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    const Plan plan = make_plan(alpha, W, offsets, K);
    const bool want_dalpha = (dalpha != nullptr || dtheta != nullptr);
    if (want_dalpha && plan.any_integral)
        return fail(FIBATTN_ERR_UNSUPPORTED,
                    "d(alpha) requested but some alpha * f_k is integral (no two-sided slope there)");

    char* ws = static_cast<char*>(workspace);
    BwdArgs a{};
    a.krot = reinterpret_cast<float*>(ws);
    ws += krot_bytes(B, L, Hkv);
    a.qrot = reinterpret_cast<float*>(ws);
    ws += align256(static_cast<size_t>(B) * Hq * L * kD * sizeof(float));
    const int S = W + 1 + plan.n_keep;
    const size_t slot_bytes = align256(static_cast<size_t>(B) * Hq * (static_cast<size_t>(W) + 1 + K) * L * sizeof(float));
    a.pbuf = reinterpret_cast<float*>(ws);
    ws += slot_bytes;
    a.dsbuf = reinterpret_cast<float*>(ws);
    ws += slot_bytes;
    a.partial = reinterpret_cast<float*>(ws);
    a.q = q;
    a.v = v;
    a.o = nullptr;
    a.lse = nullptr;
    a.dout = dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dalpha = dalpha;
    a.dtheta = dtheta;
    a.B = B;
    a.L = L;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.W = W;
    a.n_off = plan.n_keep;
    a.S = S;
    a.n_wg = bwd_query_workgroups(B, L, Hkv, Hq / Hkv);
    a.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(kD)));
    a.dalpha_dtheta = static_cast<float>(dalpha_dtheta);
    a.fr = make_freq(rope_theta);
    std::memcpy(a.off, plan.keep, sizeof(plan.keep));
    a.scan = rung_scan(plan);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (dtype == FIBATTN_BF16) {
        // matrix-core path: staged fp16 rows (the forward's layout)
        a.qscale = score_scale();
        a.xcd_map = 0;
        if (bwd_mfma_supported(a)) {
            const BwdFastLayout f = bwd_fast_layout(B, L, Hq, Hkv);
            char* w0 = static_cast<char*>(workspace);
            PrepArgs pa;
            pa.k = k;
            pa.v = v;
            pa.k16 = reinterpret_cast<_Float16*>(w0);
            pa.v16 = reinterpret_cast<_Float16*>(w0 + half_rows_bytes(B, L, Hkv));
            pa.cs = reinterpret_cast<float*>(w0 + krot_bytes(B, L, Hkv));
            pa.n_bh = B * Hkv;
            pa.L = L;
            pa.fr = a.fr;
            pa.main = 1;
            pa.k16lo = nullptr;
            pa.flags = flags_at(w0, B, L, Hkv);
            pa.n_blk = flag_blocks(L);
            a.kvflags = pa.flags;
            a.n_blk = pa.n_blk;
            a.k = k;
            a.kstage = pa.k16;
            a.vstage = pa.v16;
            a.kstage_lo = w0 + f.klo;
            a.cstab = pa.cs;
            a.qrot16 = w0 + f.qrot;
            a.do16 = w0 + f.do16;
            a.wwin = reinterpret_cast<uint32_t*>(w0 + f.wwin);
            a.wrung = reinterpret_cast<uint32_t*>(w0 + f.wrung);
            a.partial = reinterpret_cast<float*>(w0 + f.part);
            a.exps = reinterpret_cast<uint32_t*>(w0 + f.exps);
            a.seqw = reinterpret_cast<uint64_t*>(w0 + f.seqw);
            // with d(alpha) requested the query stage takes precise scores, from the low parts of
            // the rotated keys as well: written with the prep when both run in this call, else
            // by a pass of their own ahead of the query stage
            if (want_dalpha && (stages & (FIBATTN_STAGE_PREP | FIBATTN_STAGE_QUERY)))
                pa.k16lo = reinterpret_cast<_Float16*>(w0 + f.klo);
            if (stages & FIBATTN_STAGE_PREP) {
                e = launch_prep_kv16(pa, s);
                if (e != hipSuccess) return hip_fail(e, "backward prep launch");
            } else if (pa.k16lo != nullptr && (stages & FIBATTN_STAGE_QUERY)) {
                pa.main = 0;
                e = launch_prep_kv16(pa, s);
                if (e != hipSuccess) return hip_fail(e, "key low-part launch");
            }
            if (stages & (FIBATTN_STAGE_QUERY | FIBATTN_STAGE_KEY)) {
                e = launch_bwd_mfma(a, want_dalpha, stages, s);
                if (e != hipSuccess) return hip_fail(e, "bwd launch");
            }
            return FIBATTN_OK;
        }
    }

    RopeKeysArgs r;
    r.k = k;
    r.krot = const_cast<float*>(a.krot);
    r.n_bh = B * Hkv;
    r.L = L;
    r.fr = a.fr;
    if (stages & FIBATTN_STAGE_PREP) {
        e = launch_rope_keys(dtype, r, s);
        if (e != hipSuccess) return hip_fail(e, "rope_keys launch");
    }
    if (stages & (FIBATTN_STAGE_QUERY | FIBATTN_STAGE_KEY)) {
        e = launch_bwd(dtype, a, want_dalpha, stages, s);
        if (e != hipSuccess) return hip_fail(e, "bwd launch");
    }
    return FIBATTN_OK;
}

fibattn_status_t fibattn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, double alpha, int32_t W, const int32_t* offsets, int32_t K,
                             int32_t B, int32_t L, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                             double rope_theta, double dalpha_dtheta, void* dq, void* dk, void* dv, float* dalpha,
                             float* dtheta, void* workspace, size_t workspace_bytes, void* stream) {
    (void)o;
    (void)lse;
    return fibattn_bwd_stages(FIBATTN_STAGE_ALL, q, k, v, dout, alpha, W, offsets, K, B, L, Hq, Hkv, D, dtype,
                              rope_theta, dalpha_dtheta, dq, dk, dv, dalpha, dtheta, workspace, workspace_bytes,
                              stream);
}

}  // extern "C"
