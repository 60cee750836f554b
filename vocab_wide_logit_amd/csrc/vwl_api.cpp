// C ABI of the verify / fusion library: argument checks, workspace sizing,
// launch plans and dispatch.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <algorithm>
#include <atomic>
#include <mutex>

#include "vwl.h"
#include "vwl_internal.hpp"

using namespace vwl;

namespace vwl {

hipError_t launch_asym(int dt, int ds, int gate, const Plan &plan, const AsymParams &p, hipStream_t s,
                              hipEvent_t after_rows) {
    switch (ds) {
    case kDeltaAMinusB: return launch_asym_ds<kDeltaAMinusB>(dt, gate, plan, p, s, after_rows);
    case kDeltaA: return launch_asym_ds<kDeltaA>(dt, gate, plan, p, s, after_rows);
    case kDeltaTMinusB: return launch_asym_ds<kDeltaTMinusB>(dt, gate, plan, p, s, after_rows);
    }
    return hipErrorInvalidValue;
}

int asym_blocks_per_cu(int dt, int nv, int ds, int gate) {
    switch (ds) {
    case kDeltaAMinusB: return asym_blocks_per_cu_ds<kDeltaAMinusB>(dt, nv, gate);
    case kDeltaA: return asym_blocks_per_cu_ds<kDeltaA>(dt, nv, gate);
    case kDeltaTMinusB: return asym_blocks_per_cu_ds<kDeltaTMinusB>(dt, nv, gate);
    case kDeltaNone: return asym_blocks_per_cu_ds<kDeltaNone>(dt, nv, gate);
    }
    return 0;
}

} // namespace vwl

namespace {

constexpr int kNvChoices[4] = {1, 2, 4, 8};

int elem_bytes(int dt) { return dt == VWL_BF16 ? 2 : 4; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device cache of the CU count and the resident workgroups per CU of
// every kernel instance.
struct DeviceInfo {
    bool ready = false;
    int cus = 0;
    int asym_bpc[2][4][4][2] = {}; // [dtype][nv][delta source or kDeltaNone][gate]
    int rapid_bpc[2][4] = {};
    int lm_bpc = 0, lm_bpc3 = 0; // LM-head pass workgroups per CU: 64-row, 192-row
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Plan overrides for tuning sweeps (0 = automatic).
// Atomics, so a hook called while another thread plans a call is no data race.
std::atomic<int> g_force_nv[2] = {0, 0};
std::atomic<int> g_force_teams[2] = {0, 0};
std::atomic<int> g_xfam_general{0}, g_xfam_segs{0}; // cross-family verifier pass overrides
std::atomic<hipEvent_t> g_phase_event{nullptr};

const DeviceInfo *device_info() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_dev_mu);
    DeviceInfo &d = g_dev[dev];
    if (!d.ready) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            return nullptr;
        d.cus = cus;
        for (int dt = 0; dt < 2; ++dt)
            for (int k = 0; k < 4; ++k) {
                for (int ds = 0; ds < 4; ++ds)
                    for (int g = 0; g < 2; ++g)
                        d.asym_bpc[dt][k][ds][g] = asym_blocks_per_cu(dt, kNvChoices[k], ds, g);
                d.rapid_bpc[dt][k] = rapid_blocks_per_cu(dt, kNvChoices[k]);
            }
        d.lm_bpc = lmhead_blocks_per_cu(1);
        d.lm_bpc3 = lmhead_blocks_per_cu(3);
        d.ready = true;
    }
    return &d;
}

// Team size for `nv` vectors per lane: enough members (of `lanes` lanes
// each) to hold the row.
int team_size(int V, int dt, int nv, int lanes) {
    const long long per_vec = 16 / elem_bytes(dt);
    const long long nb = (V + per_vec - 1) / per_vec + 1; // body vectors, upper bound
    const long long cap = (long long)lanes * nv;
    long long w = (nb + cap - 1) / cap;
    if (w < 1)
        w = 1;
    return (int)w;
}

// Launch plan: among the vector-per-lane choices, the one of least cost (see
// below) at full residency.  Teams are then evened out over rounds.
// Every member of the grid is resident at once, so no team waits on a
// member that cannot start.
bool make_plan(int mode, int dt, long long R, int V, Plan &plan, int ds = 0, int gate = 0) {
    const DeviceInfo *d = device_info();
    if (!d)
        return false;
    // Cost of an AsymSpec plan in vector-steps per member: rounds of rows per
    // team times (the vectors a member handles per row + 4 for the per-row
    // team work), plus W/8 for the team's exchange.  Measured on the bench
    // shapes, fewest rounds alone chose 8 vectors where 4 are faster
    // (two-tensor pass at B = 64, single requests).  RAPID's row kernel keeps
    // the fewest rounds (8 vectors at its bench shape; 4 are 12% slower).
    // Ties go to more vectors.
    long long best_rounds = -1;
    double best_cost = 0.0;
    Plan best{};
    for (int k = 0; k < 4; ++k) {
        const int nv = kNvChoices[k];
        const int force_nv = g_force_nv[mode].load(std::memory_order_relaxed);
        if (force_nv && nv != force_nv)
            continue;
        const int bpc = mode == 0 ? d->asym_bpc[dt][k][ds][gate] : d->rapid_bpc[dt][k];
        if (bpc <= 0)
            continue;
        const int lanes = mode == 0 ? kAsymLanes : kRapidLanes;
        const int W = team_size(V, dt, nv, lanes);
        const long long capacity = (long long)bpc * d->cus * (kThreads / lanes); // members
        long long teams = capacity / W;
        if (teams < 1)
            continue;
        if (teams > R)
            teams = R;
        const int force_teams = g_force_teams[mode].load(std::memory_order_relaxed);
        if (force_teams > 0 && force_teams < teams)
            teams = force_teams;
        const long long rounds = (R + teams - 1) / teams;
        const double cost = mode == 0 ? (double)rounds * (nv + 4) + W / 8.0 : (double)rounds;
        if (best_rounds < 0 || cost < best_cost || (cost == best_cost && nv > best.nv)) {
            best_rounds = rounds;
            best_cost = cost;
            best.nv = nv;
            best.W = W;
            best.n_teams = (int)((R + rounds - 1) / rounds);
        }
    }
    if (best_rounds < 0)
        return false;
    const long long members = (long long)best.n_teams * best.W;
    const int per_wg = kThreads / (mode == 0 ? kAsymLanes : kRapidLanes);
    best.grid = (int)((members + per_wg - 1) / per_wg);
    plan = best;
    return true;
}

bool finite_f(float x) { return std::isfinite(x); }

static_assert(VWL_RAPID_MAX_V == kRapidMaxV, "RAPID vocabulary limit out of step with the tail geometry");
static_assert(VWL_MAX_K == kMaxDrafts, "draft limit out of step with the tail's per-row slots");

// Vectors per member: the widest row body (no head) split evenly over W.
int member_chunk(int V, int dt, int W) {
    const int per_vec = 16 / elem_bytes(dt);
    const long long nb = V / per_vec;
    const long long c = (nb + W - 1) / W;
    return (int)(c < 1 ? 1 : c);
}

// Scratch of asym_verify_noalloc: the AsymSpec workspace of one call, in a
// file-scope device array instead of caller memory.  Each device holds its
// own copy until the process ends.  The host may use its device address
// only (from hipGetSymbolAddress, once per device); the array's name in
// host code is a stand-in, not that address.
constexpr size_t kScratchBytes = VWL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

} // namespace

static vwl_status asym_variant_impl(const void *a, const void *b, const void *t, const int32_t *draft,
                                    int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                                    vwl_delta_source delta, vwl_gate gate,
                                    float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                                    int32_t *accept_len, int32_t *token, int32_t *dev_err,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

// The current device's scratch address.  The first call on a device looks the
// address up and zero-fills the array with a fill kernel on `stream` (the
// workspace contract: zero before its first use; every completed call leaves
// its counters at zero again).  No allocation.
static vwl_status scratch_for_device(hipStream_t stream, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return VWL_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return VWL_ERR_HIP;
        if (launch_fill_zero(p, kScratchBytes, stream) != hipSuccess)
            return VWL_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return VWL_OK;
}

extern "C" {

const char *vwl_status_string(int status) {
    switch (status) { // an int: a C caller may pass any value
    case VWL_OK: return "VWL_OK";
    case VWL_ERR_NULL: return "VWL_ERR_NULL: a required pointer is null";
    case VWL_ERR_SHAPE: return "VWL_ERR_SHAPE: B, K/G or V out of range";
    case VWL_ERR_DTYPE: return "VWL_ERR_DTYPE: unknown dtype";
    case VWL_ERR_PARAM: return "VWL_ERR_PARAM: beta, gamma, eta or T out of range";
    case VWL_ERR_WORKSPACE: return "VWL_ERR_WORKSPACE: workspace too small";
    case VWL_ERR_HIP: return "VWL_ERR_HIP: HIP runtime or launch failure";
    case VWL_ERR_ALIGN: return "VWL_ERR_ALIGN: a pointer is not aligned as required";
    case VWL_ERR_SCRATCH:
        return "VWL_ERR_SCRATCH: the shape needs more workspace than asym_verify_noalloc's 16 MiB scratch";
    }
    return "unknown vwl_status";
}

int vwl_version(void) { return 100; }

vwl_status vwl_workspace_reset(void *workspace, size_t bytes, hipStream_t stream) {
    if (bytes == 0)
        return VWL_OK;
    if (!workspace)
        return VWL_ERR_NULL;
    if (!aligned(workspace, 4))
        return VWL_ERR_ALIGN;
    return launch_fill_zero(workspace, bytes, stream) == hipSuccess ? VWL_OK : VWL_ERR_HIP;
}

static bool shape_ok(int B, int K, int V) {
    if (B < 1 || K < 0 || K > VWL_MAX_K || V < 1)
        return false;
    const long double n = (long double)B * (long double)(K + 1) * (long double)V;
    return n < 9.0e18L && (long long)B * (K + 1) < (1LL << 31);
}

size_t vwl_asym_workspace_bytes(int B, int K, int V, vwl_dtype dt) {
    if (!shape_ok(B, K, V) || (dt != VWL_F32 && dt != VWL_BF16))
        return 0;
    return ws_layout(B, K + 1, V, elem_bytes(dt), false).total;
}

size_t vwl_rapid_workspace_bytes(int B, int G, int V, vwl_dtype dt) {
    if (!shape_ok(B, G, V) || (dt != VWL_F32 && dt != VWL_BF16))
        return 0;
    return ws_layout(B, G + 1, V, elem_bytes(dt), true).total;
}

// The checks of an AsymSpec call; `need_a` is false only for the variant
// that never reads a (fixed gate, delta = t - b).
static vwl_status asym_check_impl(bool need_a, const void *a, const void *b, const void *t, const int32_t *draft,
                                  int B, int K, int V, int dt, float beta, float gamma,
                                  const void *D, const void *gamma_eff, const void *accept,
                                  const void *fused, const void *accept_len, const void *token,
                                  const void *workspace, size_t workspace_bytes, size_t needed_bytes) {
    if ((need_a && !a) || !b || !t || !D || !gamma_eff || !fused || !accept_len || !token)
        return VWL_ERR_NULL;
    if (K > 0 && (!draft || !accept))
        return VWL_ERR_NULL;
    if (!shape_ok(B, K, V))
        return VWL_ERR_SHAPE;
    if (dt != VWL_F32 && dt != VWL_BF16)
        return VWL_ERR_DTYPE;
    if (!finite_f(beta) || !finite_f(gamma) || gamma < 0.0f)
        return VWL_ERR_PARAM;
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(t, 16) || !aligned(D, 4) || !aligned(gamma_eff, 4) ||
        !aligned(fused, 4) || !aligned(accept_len, 4) || !aligned(token, 4) || (draft && !aligned(draft, 4)))
        return VWL_ERR_ALIGN;
    if (!workspace || workspace_bytes < needed_bytes)
        return VWL_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return VWL_ERR_ALIGN;
    return VWL_OK;
}

vwl_status vwl_asym_check(const void *a, const void *b, const void *t, const int32_t *draft,
                          int B, int K, int V, int dt, float beta, float gamma,
                          const void *D, const void *gamma_eff, const void *accept,
                          const void *fused, const void *accept_len, const void *token,
                          const void *workspace, size_t workspace_bytes, size_t needed_bytes) {
    return asym_check_impl(true, a, b, t, draft, B, K, V, dt, beta, gamma, D, gamma_eff, accept, fused, accept_len,
                           token, workspace, workspace_bytes, needed_bytes);
}

vwl_status vwl_rapid_check(const void *z, const void *y, const int32_t *draft,
                           const float *u_accept, const float *u_sample,
                           int B, int G, int V, int dt, float eta, float T,
                           const void *accept, const void *accept_len, const void *token,
                           const void *workspace, size_t workspace_bytes, size_t needed_bytes) {
    if (!z || !y || !u_sample || !accept_len || !token)
        return VWL_ERR_NULL;
    if (G > 0 && (!draft || !u_accept || !accept))
        return VWL_ERR_NULL;
    if (!shape_ok(B, G, V) || V > VWL_RAPID_MAX_V)
        return VWL_ERR_SHAPE;
    if (dt != VWL_F32 && dt != VWL_BF16)
        return VWL_ERR_DTYPE;
    if (!finite_f(eta) || eta < 0.0f || !finite_f(T) || !(T > 0.0f))
        return VWL_ERR_PARAM;
    if (!aligned(z, 16) || !aligned(y, 16) || !aligned(u_sample, 4) || !aligned(accept_len, 4) ||
        !aligned(token, 4) || (draft && !aligned(draft, 4)) || (u_accept && !aligned(u_accept, 4)))
        return VWL_ERR_ALIGN;
    if (!workspace || workspace_bytes < needed_bytes)
        return VWL_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return VWL_ERR_ALIGN;
    return VWL_OK;
}

vwl_status vwl_plan_info(int mode, int B, int K, int V, vwl_dtype dt, int64_t out[6]) {
    if (!out)
        return VWL_ERR_NULL;
    if (mode != 0 && mode != 1)
        return VWL_ERR_PARAM;
    if (!shape_ok(B, K, V))
        return VWL_ERR_SHAPE;
    if (dt != VWL_F32 && dt != VWL_BF16)
        return VWL_ERR_DTYPE;
    Plan plan;
    const long long R = (long long)B * (K + 1);
    if (!make_plan(mode, dt, R, V, plan))
        return VWL_ERR_HIP;
    out[0] = plan.W;
    out[1] = plan.nv;
    out[2] = plan.n_teams;
    out[3] = plan.grid;
    out[4] = kThreads;
    out[5] = R;
    return VWL_OK;
}

vwl_status vwl_asym_plan_info(int B, int K, int V, vwl_dtype dt, vwl_delta_source delta, vwl_gate gate,
                              int64_t out[6]) {
    if (!out)
        return VWL_ERR_NULL;
    if ((delta != VWL_DELTA_A_MINUS_B && delta != VWL_DELTA_A && delta != VWL_DELTA_T_MINUS_B) ||
        (gate != VWL_GATE_CDA && gate != VWL_GATE_FIXED))
        return VWL_ERR_PARAM;
    if (!shape_ok(B, K, V))
        return VWL_ERR_SHAPE;
    if (dt != VWL_F32 && dt != VWL_BF16)
        return VWL_ERR_DTYPE;
    Plan plan;
    const long long R = (long long)B * (K + 1);
    if (!make_plan(0, dt, R, V, plan, (int)delta, (int)gate))
        return VWL_ERR_HIP;
    out[0] = plan.W;
    out[1] = plan.nv;
    out[2] = plan.n_teams;
    out[3] = plan.grid;
    out[4] = kThreads;
    out[5] = R;
    return VWL_OK;
}

/* Tuning hook: pin the vectors-per-thread choice (1, 2, 4 or 8) and/or cap
 * the number of teams of one mode; 0 restores the automatic plan. */
vwl_status vwl_set_plan_override(int mode, int nv, int max_teams) {
    if (mode != 0 && mode != 1)
        return VWL_ERR_PARAM;
    if (nv != 0 && nv != 1 && nv != 2 && nv != 4 && nv != 8)
        return VWL_ERR_PARAM;
    if (max_teams < 0)
        return VWL_ERR_PARAM;
    g_force_nv[mode] = nv;
    g_force_teams[mode] = max_teams;
    return VWL_OK;
}

/* Tuning and test hook of asym_verify_xfam: general = 1 forces the general
 * verifier pass; segs (1..16) pins the staged pass's segment count; 0 = automatic. */
vwl_status vwl_set_xfam_override(int general, int segs) {
    if (general != 0 && general != 1)
        return VWL_ERR_PARAM;
    if (segs < 0 || segs > kXfamMaxSegs)
        return VWL_ERR_PARAM;
    g_xfam_general = general;
    g_xfam_segs = segs;
    return VWL_OK;
}

vwl_status vwl_set_phase_event(void *hip_event) {
    g_phase_event.store(static_cast<hipEvent_t>(hip_event));
    return VWL_OK;
}

vwl_status asym_verify_variant(const void *a, const void *b, const void *t, const int32_t *draft,
                               int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                               vwl_delta_source delta, vwl_gate gate,
                               float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                               int32_t *accept_len, int32_t *token, int32_t *dev_err,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return asym_variant_impl(a, b, t, draft, B, K, V, dt, beta, gamma, delta, gate, D, gamma_eff, accept, fused,
                             accept_len, token, dev_err, workspace, workspace_bytes, stream);
}

vwl_status asym_verify(const void *a, const void *b, const void *t, const int32_t *draft,
                       int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                       float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                       int32_t *accept_len, int32_t *token, int32_t *dev_err,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return asym_verify_variant(a, b, t, draft, B, K, V, dt, beta, gamma, VWL_DELTA_A_MINUS_B, VWL_GATE_CDA, D,
                               gamma_eff, accept, fused, accept_len, token, dev_err, workspace, workspace_bytes,
                               stream);
}

vwl_status asym_verify_noalloc(const void *a, const void *b, const void *t, const int32_t *draft,
                               int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                               float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                               int32_t *accept_len, int32_t *token, int32_t *dev_err, hipStream_t stream) {
    const size_t need = vwl_asym_workspace_bytes(B, K, V, dt);
    if (need > kScratchBytes)
        return VWL_ERR_SCRATCH;
    void *ws = nullptr;
    const vwl_status st = scratch_for_device(stream, &ws);
    if (st != VWL_OK)
        return st;
    // need == 0 (bad shape or dtype) is reported by the checks, in their order
    return asym_variant_impl(a, b, t, draft, B, K, V, dt, beta, gamma, VWL_DELTA_A_MINUS_B, VWL_GATE_CDA, D,
                             gamma_eff, accept, fused, accept_len, token, dev_err, ws, kScratchBytes, stream);
}

} // extern "C"

static vwl_status asym_variant_impl(const void *a, const void *b, const void *t, const int32_t *draft,
                                    int B, int K, int V, vwl_dtype dt, float beta, float gamma,
                                    vwl_delta_source delta, vwl_gate gate,
                                    float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                                    int32_t *accept_len, int32_t *token, int32_t *dev_err,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (delta != VWL_DELTA_A_MINUS_B && delta != VWL_DELTA_A && delta != VWL_DELTA_T_MINUS_B)
        return VWL_ERR_PARAM;
    if (gate != VWL_GATE_CDA && gate != VWL_GATE_FIXED)
        return VWL_ERR_PARAM;
    // a is read unless the gate is fixed and the fusion source is t - b
    const bool need_a = gate == VWL_GATE_CDA || delta != VWL_DELTA_T_MINUS_B;
    const size_t need = vwl_asym_workspace_bytes(B, K, V, dt);
    const vwl_status st = asym_check_impl(need_a, a, b, t, draft, B, K, V, (int)dt, beta, gamma, D, gamma_eff,
                                          accept, fused, accept_len, token, workspace, workspace_bytes, need);
    if (st != VWL_OK)
        return st;
    if (dev_err && !aligned(dev_err, 4))
        return VWL_ERR_ALIGN;
    const long long R = (long long)B * (K + 1);
    Plan plan;
    if (!make_plan(0, (int)dt, R, V, plan, (int)delta, (int)gate))
        return VWL_ERR_HIP;
    const WsLayout L = ws_layout(B, K + 1, V, elem_bytes(dt), false);
    char *ws = static_cast<char *>(workspace);
    AsymParams p{};
    p.a = a;
    p.b = b;
    p.t = t;
    p.draft = draft;
    p.R = R;
    p.B = B;
    p.K = K;
    p.V = V;
    p.W = plan.W;
    p.n_teams = plan.n_teams;
    p.Wmax = L.Wmax;
    p.chunk = member_chunk(V, (int)dt, plan.W);
    p.beta = beta;
    p.gamma = gamma;
    p.log_gamma = std::log((double)gamma);
    p.D = D;
    p.geff = gamma_eff;
    p.accept = accept;
    p.fused = fused;
    p.acc_len = accept_len;
    p.token = token;
    p.dev_err = dev_err;
    p.ctl = reinterpret_cast<uint32_t *>(ws + L.ctl);
    p.rec = reinterpret_cast<uint64_t *>(ws + L.rec);
    p.lsum = reinterpret_cast<uint64_t *>(ws + L.lsum);
    return launch_asym((int)dt, (int)delta, (int)gate, plan, p, stream, g_phase_event.load()) == hipSuccess
               ? VWL_OK
               : VWL_ERR_HIP;
}

extern "C" {

// Cross-family workspace: the AsymSpec layout of the drafter rows, the
// verifier records (enough for either verifier pass), then the per-part
// inverse alignment of the staged pass and its flag.
static bool xfam_layout(int B, int K, int Vd, int Vt, vwl_dtype dt, WsLayout &L, size_t &vrec, size_t &xkey,
                        size_t &total) {
    if (!shape_ok(B, K, Vd) || !shape_ok(B, K, Vt) || (dt != VWL_F32 && dt != VWL_BF16))
        return false;
    const long long R = (long long)B * (K + 1);
    const long long C = std::max<long long>(xfam_chunks(Vt), (long long)xfam_parts(Vt, elem_bytes(dt)) * kXfamMaxSegs);
    if (8 * ((R + 7) / 8) * C > 0x7fffffffLL) // workgroups of the verifier pass
        return false;
    L = ws_layout(B, K + 1, Vd, elem_bytes(dt), false);
    vrec = L.total;
    xkey = align256(vrec + (size_t)R * C * kVrecWords * 8);
    // xkey[parts][Vd], then the flag word
    total = align256(xkey + (xfam_key_words(xfam_parts(Vt, elem_bytes(dt)), Vd) + 1) * 4);
    return true;
}

// Geometry of the staged verifier pass, or false when the general pass runs:
// the rows must be made of whole 16-byte vectors (the row pointers are
// 16-byte aligned by the argument checks; rechecked here).  Parts: the fewest of at most xfam_part_cap tokens, of equal
// length (a multiple of 8 tokens).  Segments: the count (up to kXfamMaxSegs) that
// minimises rounds of resident workgroups (one per CU) times the bytes one
// workgroup moves (its part plus its segment's a, b and inverse alignment).
static bool xfam_staged_geometry(const void *a, const void *b, const void *t, int Vd, int Vt, int dt, long long R,
                                 int cus, AsymParams &p) {
    const int eb = elem_bytes(dt);
    const int force_segs = g_xfam_segs.load(std::memory_order_relaxed);
    if (g_xfam_general.load(std::memory_order_relaxed) || !aligned(a, 16) || !aligned(b, 16) || !aligned(t, 16) || ((long long)Vd * eb) % 16 ||
        ((long long)Vt * eb) % 16)
        return false;
    const int parts = xfam_parts(Vt, eb);
    const int partlen = (int)((((long long)Vt + parts - 1) / parts + 7) / 8 * 8);
    if (partlen > xfam_part_cap(eb) || (long long)(parts - 1) * partlen >= Vt)
        return false;
    int best_s = 1;
    double best_cost = 0.0;
    for (int sg = 1; sg <= kXfamMaxSegs; ++sg) {
        if (force_segs && sg != force_segs)
            continue;
        const long long seglen = (((long long)Vd + sg - 1) / sg + 7) / 8 * 8;
        const long long rounds = (8 * ((R + 7) / 8) * parts * sg + cus - 1) / cus;
        const double cost = (double)rounds * ((double)partlen * eb + (double)seglen * (2.0 * eb + 2.0));
        if (sg == 1 || force_segs || cost < best_cost) {
            best_cost = cost;
            best_s = sg;
        }
    }
    p.xparts = parts;
    p.xpartlen = partlen;
    p.xsegs = best_s;
    p.xseglen = (int)((((long long)Vd + best_s - 1) / best_s + 7) / 8 * 8);
    p.xsharelen = (int)((((long long)partlen + best_s - 1) / best_s + 7) / 8 * 8);
    p.vchunks = parts * best_s;
    return true;
}

size_t vwl_asym_xfam_workspace_bytes(int B, int K, int Vd, int Vt, vwl_dtype dt) {
    WsLayout L;
    size_t vrec, xkey, total;
    return xfam_layout(B, K, Vd, Vt, dt, L, vrec, xkey, total) ? total : 0;
}

vwl_status asym_verify_xfam(const void *a, const void *b, int Vd, const void *t, int Vt, const int32_t *vmap,
                            const int32_t *draft, int B, int K, vwl_dtype dt, float beta, float gamma,
                            float *D, float *gamma_eff, uint8_t *accept, int32_t *fused,
                            int32_t *accept_len, int32_t *token, int32_t *dev_err,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!vmap)
        return VWL_ERR_NULL;
    if (Vt < 1)
        return VWL_ERR_SHAPE;
    const size_t need = vwl_asym_xfam_workspace_bytes(B, K, Vd, Vt, dt);
    // the same checks as asym_verify on the drafter shape, then the verifier's
    const vwl_status st = asym_check_impl(true, a, b, t, draft, B, K, Vd, (int)dt, beta, gamma, D, gamma_eff,
                                          accept, fused, accept_len, token, workspace, workspace_bytes,
                                          need ? need : 1);
    if (st != VWL_OK)
        return st;
    WsLayout L;
    size_t vrec, xkey, total;
    if (!xfam_layout(B, K, Vd, Vt, dt, L, vrec, xkey, total))
        return VWL_ERR_SHAPE;
    if (!aligned(vmap, 4) || (dev_err && !aligned(dev_err, 4)))
        return VWL_ERR_ALIGN;
    const long long R = (long long)B * (K + 1);
    Plan plan;
    if (!make_plan(0, (int)dt, R, Vd, plan, kDeltaNone, kGateCda))
        return VWL_ERR_HIP;
    const DeviceInfo *dev = device_info();
    if (!dev)
        return VWL_ERR_HIP;
    char *ws = static_cast<char *>(workspace);
    AsymParams p{};
    p.a = a;
    p.b = b;
    p.t = nullptr;
    p.tv = t;
    p.Vt = Vt;
    if (!xfam_staged_geometry(a, b, t, Vd, Vt, (int)dt, R, dev->cus, p)) {
        p.xparts = 0;
        p.vchunks = xfam_chunks(Vt);
    }
    p.vmap = vmap;
    p.vrec = reinterpret_cast<uint64_t *>(ws + vrec);
    p.xkey = reinterpret_cast<uint16_t *>(ws + xkey);
    p.xdup = reinterpret_cast<uint32_t *>(ws + xkey) + xfam_key_words(xfam_parts(Vt, elem_bytes(dt)), Vd);
    p.draft = draft;
    p.R = R;
    p.B = B;
    p.K = K;
    p.V = Vd;
    p.W = plan.W;
    p.n_teams = plan.n_teams;
    p.Wmax = L.Wmax;
    p.chunk = member_chunk(Vd, (int)dt, plan.W);
    p.beta = beta;
    p.gamma = gamma;
    p.log_gamma = std::log((double)gamma);
    p.D = D;
    p.geff = gamma_eff;
    p.accept = accept;
    p.fused = fused;
    p.acc_len = accept_len;
    p.token = token;
    p.dev_err = dev_err;
    p.ctl = reinterpret_cast<uint32_t *>(ws + L.ctl);
    p.rec = reinterpret_cast<uint64_t *>(ws + L.rec);
    p.lsum = reinterpret_cast<uint64_t *>(ws + L.lsum);
    return launch_xfam((int)dt, plan, p, stream, g_phase_event.load()) == hipSuccess ? VWL_OK : VWL_ERR_HIP;
}

// LM-head pass geometry: row tiles of kLmRowTile, vocabulary ranges
// (multiples of 128 tokens) and the JSD pass's chunks.
struct LmGeom {
    int G, RT, S, range, jc;
    long long lgs;
    size_t rec, rowstat, lg, jpart, total_min, total;
};
// Shapes and workspace layout.  The records hold one entry per (row,
// vocabulary range) for up to one range per 128-column tile, so the size
// does not depend on the device; lm_split picks the ranges at launch.  The
// JSD partials are sized for either JSD pass (one per 4096 tokens or one per
// range), and the stored pairs come last: a workspace of total_min bytes
// runs the path with no pair storage.  Every launch's work-items must number
// below 2^32.
static bool lm_geometry(int B, int K, int V, int Hd, int Ht, LmGeom &g) {
    if (!shape_ok(B, K, V) || Hd < 64 || Ht < 64 || Hd % 64 || Ht % 64)
        return false;
    const long long R = (long long)B * (K + 1);
    // past 128 rows a workgroup takes 192 rows (3 groups of 4 waves sharing
    // each head tile), else 64
    const int G = R > 2 * kLmRowTile ? 3 : 1;
    const long long RT = (R + G * kLmRowTile - 1) / (G * kLmRowTile);
    const long long max_wgs = 0xffffffffLL / (kThreads * G);
    if (RT > (1LL << 24))
        return false;
    const long long tiles = ((long long)V + 127) / 128;
    if (8 * RT * ((tiles + 7) / 8) > max_wgs)
        return false;
    const long long jc = ((long long)V + kLmJsdChunk - 1) / kLmJsdChunk;
    if (R * jc > max_wgs)
        return false;
    // the stored pairs cover whole tiles: RT * 64 G rows of whole 128-token tiles
    const long long lgs = tiles * 128;
    if ((long double)(RT * G * kLmRowTile) * (long double)lgs * 8.0L > 4.0e18L)
        return false;
    g.G = G;
    g.RT = (int)RT;
    g.S = (int)tiles;
    g.range = 128;
    g.jc = (int)jc;
    g.lgs = lgs;
    size_t off = 0;
    g.rec = off;      off = align256(off + (size_t)R * tiles * kRecWords * 8);
    g.rowstat = off;  off = align256(off + (size_t)R * kLmStat * 8);
    g.jpart = off;    off = align256(off + (size_t)R * (size_t)(tiles > jc ? tiles : jc) * 8);
    g.total_min = off;
    g.lg = off;       off = align256(off + (size_t)(RT * G * kLmRowTile) * (size_t)lgs * 8);
    g.total = off;
    return true;
}

// Vocabulary ranges of whole 128-column tiles for `capacity` resident
// workgroups: the split that finishes in the fewest tile steps, counting the
// rounds of workgroups the grid needs (8 x RT x ceil(S / 8) workgroups with
// the die-aware numbering); ties go to the finer split.
static void lm_split(LmGeom &g, int V, long long capacity) {
    const long long tiles = ((long long)V + 127) / 128;
    long long best_cost = -1, best_r = 1;
    for (long long r = 1; r <= tiles; ++r) {
        const long long S = (tiles + r - 1) / r;
        const long long grid = 8 * (long long)g.RT * ((S + 7) / 8);
        const long long rounds = capacity > 0 ? (grid + capacity - 1) / capacity : 1;
        const long long cost = rounds * r;
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_r = r;
        }
    }
    g.range = (int)(best_r * 128);
    g.S = (int)(((long long)V + g.range - 1) / g.range);
}

size_t vwl_asym_lmhead_workspace_bytes(int B, int K, int V, int Hd, int Ht) {
    LmGeom g;
    return lm_geometry(B, K, V, Hd, Ht, g) ? g.total : 0;
}

size_t vwl_asym_lmhead_workspace_min_bytes(int B, int K, int V, int Hd, int Ht) {
    LmGeom g;
    return lm_geometry(B, K, V, Hd, Ht, g) ? g.total_min : 0;
}

vwl_status asym_verify_lmhead(const void *h_a, const void *h_b, const void *W_d, const void *h_t, const void *W_t,
                              const int32_t *draft, int B, int K, int V, int Hd, int Ht, float beta, float gamma,
                              float *D, float *gamma_eff, uint8_t *accept, int32_t *fused, int32_t *accept_len,
                              int32_t *token, int32_t *dev_err, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    if (!h_a || !h_b || !W_d || !h_t || !W_t || !D || !gamma_eff || !fused || !accept_len || !token)
        return VWL_ERR_NULL;
    if (K > 0 && (!draft || !accept))
        return VWL_ERR_NULL;
    LmGeom g;
    if (!lm_geometry(B, K, V, Hd, Ht, g))
        return VWL_ERR_SHAPE;
    if (!finite_f(beta) || !finite_f(gamma) || gamma < 0.0f)
        return VWL_ERR_PARAM;
    const DeviceInfo *dev = device_info();
    if (!dev)
        return VWL_ERR_HIP;
    lm_split(g, V, (long long)dev->cus * (g.G == 3 ? dev->lm_bpc3 : dev->lm_bpc));
    if (!aligned(h_a, 16) || !aligned(h_b, 16) || !aligned(W_d, 16) || !aligned(h_t, 16) || !aligned(W_t, 16) ||
        !aligned(D, 4) || !aligned(gamma_eff, 4) || !aligned(fused, 4) || !aligned(accept_len, 4) ||
        !aligned(token, 4) || (draft && !aligned(draft, 4)) || (dev_err && !aligned(dev_err, 4)))
        return VWL_ERR_ALIGN;
    if (!workspace || workspace_bytes < g.total_min)
        return VWL_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return VWL_ERR_ALIGN;
    const bool store = workspace_bytes >= g.total; // room for the (a, b) pairs
    char *ws = static_cast<char *>(workspace);
    LmheadParams p{};
    p.ha = static_cast<const uint16_t *>(h_a);
    p.hb = static_cast<const uint16_t *>(h_b);
    p.ht = static_cast<const uint16_t *>(h_t);
    p.Wd = static_cast<const uint16_t *>(W_d);
    p.Wt = static_cast<const uint16_t *>(W_t);
    p.draft = draft;
    p.R = (long long)B * (K + 1);
    p.B = B;
    p.K = K;
    p.V = V;
    p.Hd = Hd;
    p.Ht = Ht;
    p.G = g.G;
    p.RT = g.RT;
    p.S = g.S;
    p.range = g.range;
    p.beta = beta;
    p.gamma = gamma;
    p.log_gamma = std::log((double)gamma);
    p.D = D;
    p.geff = gamma_eff;
    p.accept = accept;
    p.fused = fused;
    p.acc_len = accept_len;
    p.token = token;
    p.dev_err = dev_err;
    p.rec = reinterpret_cast<uint64_t *>(ws + g.rec);
    p.rowstat = reinterpret_cast<double *>(ws + g.rowstat);
    p.lg = store ? reinterpret_cast<float *>(ws + g.lg) : nullptr;
    p.lgs = g.lgs;
    p.jpart = reinterpret_cast<double *>(ws + g.jpart);
    p.jc = store ? g.jc : g.S; // JSD partials per row: per 4096 tokens, or per range
    return launch_lmhead(p, stream, g_phase_event.load()) == hipSuccess ? VWL_OK : VWL_ERR_HIP;
}

size_t vwl_e2sci_workspace_bytes(int B, int W, int V, vwl_dtype dt) {
    if (W < 1 || !shape_ok(B, W - 1, V) || (dt != VWL_F32 && dt != VWL_BF16))
        return 0;
    return ws_layout(B, W, V, elem_bytes(dt), false).total;
}

vwl_status e2sci_verify(const void *y, const void *z, int B, int W, int V, vwl_dtype dt,
                        const float *T_in, const float *omega, float *r_hat, int32_t *age,
                        const vwl_e2sci_params *params,
                        float *D, uint8_t *accept, int32_t *accept_len, float *T_out,
                        int32_t *dev_err, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!y || !z || !T_in || !omega || !r_hat || !params || !D || !accept || !accept_len || !T_out)
        return VWL_ERR_NULL;
    if (W < 1 || !shape_ok(B, W - 1, V))
        return VWL_ERR_SHAPE;
    if (dt != VWL_F32 && dt != VWL_BF16)
        return VWL_ERR_DTYPE;
    const vwl_e2sci_params &q = *params;
    if (!finite_f(q.alpha) || !finite_f(q.tau_credit) || !finite_f(q.T_base) || !finite_f(q.T_min) ||
        !finite_f(q.T_max) || !(q.T_min <= q.T_max) || !(q.ewma >= 0.0f && q.ewma <= 1.0f) ||
        !finite_f(q.hysteresis) || !(q.hysteresis >= 0.0f) || q.min_refresh < 0 || !finite_f(q.delta) ||
        !finite_f(q.T_safe) || (q.delta > 0.0f && !(q.T_min <= q.T_safe && q.T_safe <= q.T_max)))
        return VWL_ERR_PARAM;
    if (q.min_refresh > 1 && !age)
        return VWL_ERR_NULL;
    if (!aligned(y, 16) || !aligned(z, 16) || !aligned(T_in, 4) || !aligned(omega, 4) || !aligned(r_hat, 4) ||
        !aligned(D, 4) || !aligned(accept_len, 4) || !aligned(T_out, 4) || (dev_err && !aligned(dev_err, 4)) ||
        (age && !aligned(age, 4)))
        return VWL_ERR_ALIGN;
    const size_t need = vwl_e2sci_workspace_bytes(B, W, V, dt);
    if (!workspace || workspace_bytes < need)
        return VWL_ERR_WORKSPACE;
    if (!aligned(workspace, 256))
        return VWL_ERR_ALIGN;
    const long long R = (long long)B * W;
    Plan plan;
    if (!make_plan(0, (int)dt, R, V, plan, kDeltaNone, kGateCda))
        return VWL_ERR_HIP;
    const WsLayout L = ws_layout(B, W, V, elem_bytes(dt), false);
    char *ws = static_cast<char *>(workspace);
    AsymParams p{};
    p.a = y;
    p.b = z;
    p.t = nullptr;
    p.R = R;
    p.B = B;
    p.K = W - 1;
    p.V = V;
    p.W = plan.W;
    p.n_teams = plan.n_teams;
    p.Wmax = L.Wmax;
    p.chunk = member_chunk(V, (int)dt, plan.W);
    p.D = D;
    p.accept = accept;
    p.acc_len = accept_len;
    p.dev_err = dev_err;
    p.ctl = reinterpret_cast<uint32_t *>(ws + L.ctl);
    p.rec = reinterpret_cast<uint64_t *>(ws + L.rec);
    p.lsum = reinterpret_cast<uint64_t *>(ws + L.lsum);
    p.win = W;
    p.thr_in = T_in;
    p.omega = omega;
    p.r_hat = r_hat;
    p.thr_out = T_out;
    p.e_alpha = q.alpha;
    p.e_tau = q.tau_credit;
    p.e_Tbase = q.T_base;
    p.e_Tmin = q.T_min;
    p.e_Tmax = q.T_max;
    p.e_ewma = q.ewma;
    p.e_hyst = q.hysteresis;
    p.e_delta = q.delta;
    p.e_Tsafe = q.T_safe;
    p.e_minref = q.min_refresh;
    p.age = age;
    return launch_e2sci((int)dt, plan, p, stream, g_phase_event.load()) == hipSuccess ? VWL_OK : VWL_ERR_HIP;
}

vwl_status vwl_e2sci_plan_info(int B, int W, int V, vwl_dtype dt, int64_t out[6]) {
    if (!out)
        return VWL_ERR_NULL;
    if (W < 1 || !shape_ok(B, W - 1, V))
        return VWL_ERR_SHAPE;
    if (dt != VWL_F32 && dt != VWL_BF16)
        return VWL_ERR_DTYPE;
    Plan plan;
    const long long R = (long long)B * W;
    if (!make_plan(0, dt, R, V, plan, kDeltaNone, kGateCda))
        return VWL_ERR_HIP;
    out[0] = plan.W;
    out[1] = plan.nv;
    out[2] = plan.n_teams;
    out[3] = plan.grid;
    out[4] = kThreads;
    out[5] = R;
    return VWL_OK;
}

vwl_status rapid_verify(const void *z, const void *y, const int32_t *draft,
                        const float *u_accept, const float *u_sample,
                        int B, int G, int V, vwl_dtype dt, float eta, float T,
                        uint8_t *accept, int32_t *accept_len, int32_t *token,
                        float *p_hat_draft, float *q_draft, float *emit_dist,
                        int32_t *dev_err, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    const size_t need = vwl_rapid_workspace_bytes(B, G, V, dt);
    const vwl_status st = vwl_rapid_check(z, y, draft, u_accept, u_sample, B, G, V, (int)dt, eta, T, accept,
                                          accept_len, token, workspace, workspace_bytes, need);
    if (st != VWL_OK)
        return st;
    if ((dev_err && !aligned(dev_err, 4)) || (p_hat_draft && !aligned(p_hat_draft, 4)) ||
        (q_draft && !aligned(q_draft, 4)) || (emit_dist && !aligned(emit_dist, 4)))
        return VWL_ERR_ALIGN;
    const long long R = (long long)B * (G + 1);
    Plan plan;
    if (!make_plan(1, (int)dt, R, V, plan))
        return VWL_ERR_HIP;
    const WsLayout L = ws_layout(B, G + 1, V, elem_bytes(dt), true);
    char *ws = static_cast<char *>(workspace);
    RapidParams p{};
    p.z = z;
    p.y = y;
    p.draft = draft;
    p.u_accept = u_accept;
    p.u_sample = u_sample;
    p.R = R;
    p.B = B;
    p.G = G;
    p.V = V;
    p.W = plan.W;
    p.n_teams = plan.n_teams;
    p.Wmax = L.Wmax;
    p.chunk = member_chunk(V, (int)dt, plan.W);
    p.We = L.We;
    p.ept = L.ept;
    {
        // log2e / T split into a high part not above it and a positive low
        // part (a -inf logit times a positive low part stays -inf)
        const double c = 1.4426950408889634 / (double)T;
        float hi = (float)c;
        if ((double)hi > c)
            hi = std::nextafter(hi, 0.0f);
        float lo = (float)(c - (double)hi);
        if (!(lo > 0.0f))
            lo = std::numeric_limits<float>::min();
        p.c_hi = hi;
        p.c_lo = lo;
        p.eta2 = (float)((double)eta * 1.4426950408889634);
    }
    p.T = (double)T;
    p.invT64 = 1.0 / (double)T;
    p.eta_d = (double)eta;
    p.accept = accept;
    p.acc_len = accept_len;
    p.token = token;
    p.dev_err = dev_err;
    p.p_hat_draft = p_hat_draft;
    p.q_draft = q_draft;
    p.emit_dist = emit_dist;
    p.ctl = reinterpret_cast<uint32_t *>(ws + L.ctl);
    p.req_ctr = reinterpret_cast<uint32_t *>(ws + L.req_ctr);
    p.rec = reinterpret_cast<uint64_t *>(ws + L.rec);
    p.rowstat = reinterpret_cast<double *>(ws + L.rowstat);
    p.emit = reinterpret_cast<double *>(ws + L.emit);
    p.xw = reinterpret_cast<uint64_t *>(ws + L.lsum);
    return launch_rapid((int)dt, plan, p, stream, g_phase_event.load()) == hipSuccess ? VWL_OK : VWL_ERR_HIP;
}

} // extern "C"
