// Internal host/device declarations: workspace layout, kernel parameter
// blocks and the launchers of each kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vwl {

constexpr int kThreads = 256; // threads per workgroup (4 wave64)

// Workspace layout (bytes, each block 256-byte aligned).  Sizes depend only on
// the call's shape, never on the device, so they can be queried on any host.
//
//   ctl      64 x u32   [0] ticket counter of the row kernel
//   req_ctr  B x 16 u32 RAPID only: per request, the tail's [4] phase
//            arrivals and [5] departures
//   rec      R x Wmax x 8 u64  per (row, member) record (see the kernels)
//   rowstat  R x 8 f64  RAPID: L_z, L_y, Mhat, L_zhat, argmax of zhat
//            R x 4 f64  AsymSpec: L_a, L_b, L_t (log2 units), fused token
//   emit     B x We x 8 f64  RAPID only: per-chunk residual, target,
//                             augmented-target and normaliser sums
//   lsum     R x Wmax x 2 u64  AsymSpec: each member's log-sum-exps of a
//            and b (log2 units), in the form lse_word() gives them
//            R x Wmax x 4 u64  RAPID: each member's sums of z and y and
//            their references as the row kernel publishes them
//            zero means "not yet published" (the finalize kernels, and the
//            RAPID tail, clear them for the next call)
struct WsLayout {
    size_t ctl, req_ctr, rec, rowstat, emit, lsum, total;
    int Wmax;
    int We;  // RAPID: workgroups per request in the tail
    int ept; // RAPID: emitting-row elements per thread in the tail
};

constexpr int kRecWords = 8;
// Threads of a per-request finalize workgroup: one wave per row, at most 16.
constexpr int kFinMaxThreads = 1024;
inline unsigned fin_threads(int rows) { return 64u * (unsigned)(rows < 16 ? (rows < 1 ? 1 : rows) : 16); }
constexpr int kEmitMaxChunks = 512; // tail workgroups per request (at most)
constexpr int kRapidMaxV = kThreads * 16 * kEmitMaxChunks; // largest RAPID vocabulary
constexpr int kRowStatWords = 8;
constexpr int kMaxDrafts = 63; // drafts per request (the API's limit)
constexpr int kEmitWords = 8;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Lanes of one team member (a whole workgroup in both modes).
constexpr int kAsymLanes = kThreads;
constexpr int kRapidLanes = kThreads;

// Largest team size any plan may use: one 16-byte vector per lane.
inline int max_team(int V, int elem_bytes, int lanes) {
    const long long per_vec = 16 / elem_bytes;
    const long long nb = (V + per_vec - 1) / per_vec + 1;
    long long w = (nb + lanes - 1) / lanes;
    return (int)(w < 1 ? 1 : w);
}

inline WsLayout ws_layout(int B, int P, int V, int elem_bytes, bool rapid) {
    WsLayout L{};
    const size_t R = (size_t)B * (size_t)P;
    L.Wmax = max_team(V, elem_bytes, rapid ? kRapidLanes : kAsymLanes);
    if (rapid) {
        // 8 elements per tail thread, 16 past 8 * 256 * kEmitMaxChunks
        L.ept = ((long long)V > (long long)kThreads * 8 * kEmitMaxChunks) ? 16 : 8;
        L.We = (int)(((long long)V + kThreads * L.ept - 1) / ((long long)kThreads * L.ept));
    }
    size_t off = 0;
    L.ctl = off;      off = align256(off + 64 * 4);
    L.req_ctr = off;  off = align256(off + (rapid ? (size_t)B * 16 * 4 : 0));
    L.rec = off;      off = align256(off + R * (size_t)L.Wmax * kRecWords * 8);
    L.rowstat = off;  off = align256(off + R * (rapid ? kRowStatWords : 4) * 8);
    L.emit = off;     off = align256(off + (rapid ? (size_t)B * (size_t)L.We * kEmitWords * 8 : 0));
    L.lsum = off;     off = align256(off + R * (size_t)L.Wmax * (rapid ? 4 : 2) * 8);
    L.total = off;
    return L;
}

struct AsymParams {
    const void *a, *b, *t;
    const int32_t *draft;
    long long R;
    int B, K, V;
    int W, n_teams, Wmax;
    int chunk;          // vectors per member (fixed per launch)
    float beta, gamma;
    double log_gamma;
    float *D, *geff;
    uint8_t *accept;
    int32_t *fused, *acc_len, *token, *dev_err;
    uint32_t *ctl;
    uint64_t *rec;
    uint64_t *lsum; // [R][Wmax][2] published log-sum-exps of a and b
    // AsymSpec across families: verifier rows on their own vocabulary Vt,
    // the alignment vmap[Vt] (paired drafter id or -1), per-(row, chunk)
    // verifier records [R][vchunks][kVrecWords].  The staged verifier pass
    // (xparts > 0) splits the verifier row into xparts parts of xpartlen
    // tokens and the drafter row into xsegs segments of xseglen tokens, with
    // xsharelen tokens of a part per segment for L_t.  It uses the inverse
    // alignment per part, xkey[xparts][Vd] (16 bits): for drafter token d
    // paired with verifier token v = p*xpartlen + i of part p, i + 1, else 0;
    // and the flag xdup (two verifier tokens of one part share a drafter
    // token), the 32-bit word after the keys.  Both are zero between calls.
    const void *tv;
    int Vt, vchunks;
    const int32_t *vmap;
    uint64_t *vrec;
    uint16_t *xkey;
    uint32_t *xdup;
    int xparts, xpartlen, xsegs, xseglen, xsharelen;
    // E2-SCI (a = drafter y, b = target z; `win` rows per request)
    int win;
    const float *thr_in, *omega;
    float *r_hat, *thr_out;
    double e_alpha, e_tau, e_Tbase, e_Tmin, e_Tmax, e_ewma;
    double e_hyst, e_delta, e_Tsafe; // stabilisers of the threshold update
    int e_minref;
    int32_t *age;                    // [B] windows in effect of each threshold, nullable
};

struct RapidParams {
    const void *z, *y;
    const int32_t *draft;
    const float *u_accept, *u_sample;
    long long R;
    int B, G, V;
    int W, n_teams, Wmax, We, ept;
    int chunk;          // vectors per member (fixed per launch)
    float c_hi, c_lo; // log2e / T = c_hi + c_lo, c_hi <= log2e / T, c_lo > 0
    float eta2;       // eta * log2e
    double T, eta_d, invT64;
    uint8_t *accept;
    int32_t *acc_len, *token, *dev_err;
    float *p_hat_draft, *q_draft, *emit_dist;
    uint32_t *ctl, *req_ctr;
    uint64_t *rec;
    double *rowstat, *emit;
    uint64_t *xw; // [R][Wmax][4] published phase-1 words of the row kernel
};

// A launch plan: vectors per thread per tensor (template choice), team size,
// number of teams (grid = n_teams * W).
struct Plan {
    int nv;
    int W;
    int n_teams;
    int grid;
};

// AsymSpec from hidden states and LM heads (bf16 throughout).
struct LmheadParams {
    const uint16_t *ha, *hb, *ht; // [R][Hd], [R][Hd], [R][Ht]
    const uint16_t *Wd, *Wt;      // [V][Hd], [V][Ht]
    const int32_t *draft;
    long long R;
    int B, K, V, Hd, Ht;
    int G;     // groups of 64 rows per workgroup (1 or 3)
    int RT;    // row tiles of 64 G
    int S;     // vocabulary ranges (records per row)
    int range; // tokens per range (a multiple of 128)
    float beta, gamma;
    double log_gamma;
    float *D, *geff;
    uint8_t *accept;
    int32_t *fused, *acc_len, *token, *dev_err;
    uint64_t *rec;    // [R][S][8], the row kernel's record layout
    double *rowstat;  // [R][kLmStat] L_a, L_b, L_t (log2 units), fused token, t_d, b_d
    float *lg;        // [RT * 64 G][lgs][2] the logit pairs (a, b) of the first launch
    long long lgs;    // pairs per row of lg (V rounded up to whole 128-token tiles)
    double *jpart;    // [R][jc] the JSD pass's partial sums
    int jc;           // JSD chunks per row
};
// Rows per workgroup of the LM-head pass (MFMA row blocks of 16).
constexpr int kLmRowTile = 64;
constexpr int kLmStat = 6; // per-row statistics of the LM-head path
// JSD pass over the stored pairs: 16 pairs per thread, so a workgroup chunk
// is 4096 tokens.
constexpr int kLmJsdPairs = 16;
constexpr int kLmJsdChunk = kThreads * kLmJsdPairs;
hipError_t launch_lmhead(const LmheadParams &p, hipStream_t s, hipEvent_t after_rows);
int lmhead_blocks_per_cu(int G);

// AsymSpec variants (values match vwl_delta_source / vwl_gate of the C ABI);
// kDeltaNone is the two-tensor divergence pass of E2-SCI.
enum { kDeltaAMinusB = 0, kDeltaA = 1, kDeltaTMinusB = 2, kDeltaNone = 3 };
enum { kGateCda = 0, kGateFixed = 1 };

// Launchers (return hipSuccess or the launch error).
// `after_rows`, when non-null, is recorded on `s` between the row kernel and
// the kernels that follow it.  The AsymSpec launcher of fusion source DS is
// instantiated in its own translation unit (asym_<delta>.hip).
template <int DS>
hipError_t launch_asym_ds(int dt, int gate, const Plan &plan, const AsymParams &p, hipStream_t s,
                          hipEvent_t after_rows);
hipError_t launch_e2sci(int dt, const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows);
hipError_t launch_xfam(int dt, const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows);

// Cross-family verifier pass: elements per thread and per workgroup chunk,
// and the record of one (row, chunk).
constexpr int kXfamEpt = 16;
constexpr int kXfamChunk = kThreads * kXfamEpt;
constexpr int kVrecWords = 4;
inline int xfam_chunks(int Vt) { return (Vt + kXfamChunk - 1) / kXfamChunk; }
// Staged verifier pass: 1024-thread workgroups, each holding one part of a
// verifier row (at most 128 KiB) in LDS; at most kXfamMaxSegs drafter
// segments per row.
constexpr int kXlThreads = 1024;
constexpr int kXlLdsVecs = 8192; // a part's 16-byte vectors, after one leading vector of -inf
constexpr int kXfamMaxSegs = 16;
// Tokens per part: what LDS holds, and below 2^16 so that i + 1 is a key.
inline int xfam_part_cap(int elem_bytes) {
    const int cap = kXlLdsVecs * 16 / elem_bytes;
    return cap < 65528 ? cap : 65528;
}
inline int xfam_parts(int Vt, int elem_bytes) {
    const int cap = xfam_part_cap(elem_bytes);
    return (Vt + cap - 1) / cap;
}
// 32-bit words of the keys of the staged pass; the flag word follows them.
__host__ __device__ inline size_t xfam_key_words(int parts, int Vd) { return ((size_t)parts * Vd + 1) / 2; }
hipError_t launch_rapid(int dt, const Plan &plan, const RapidParams &p, hipStream_t s, hipEvent_t after_rows);
hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t s);

// Resident workgroups per CU of each kernel instance (0 when unknown).
template <int DS>
int asym_blocks_per_cu_ds(int dt, int nv, int gate);
int rapid_blocks_per_cu(int dt, int nv);

// Dispatch over the fusion source (defined with the C ABI, outside the kernel
// translation units, so each of those instantiates only its own source).
hipError_t launch_asym(int dt, int ds, int gate, const Plan &plan, const AsymParams &p, hipStream_t s,
                       hipEvent_t after_rows);
int asym_blocks_per_cu(int dt, int nv, int ds, int gate);

} // namespace vwl
