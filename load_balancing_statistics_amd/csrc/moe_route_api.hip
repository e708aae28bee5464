// moe_route_api.hip -- the C ABI declared in include/moe_route.h: argument
// validation on the host, workspace sizing, and the launch sequence
//   [gate transpose + gate GEMM] -> row pass -> block scan + statistics
//   -> dispatch scatter
// for the forward (one launch after the gate GEMM for small microbatches),
// and the single streaming pass of the backward.
#include <climits>
#include <cmath>
#include <mutex>

#include "route_common.hpp"

// Scratch of moe_route_noalloc: one call's workspace in a device array the
// library owns.  The runtime gives every GPU that loads this library its own
// copy at its own address.  In host code the name is only a stand-in, never
// a device address: host code uses the per-device address that
// hipGetSymbolAddress returns (scratch_of_current_device below).
static __device__ __align__(256) unsigned char scratch[MOE_ROUTE_SCRATCH_BYTES];

namespace {

using moe::RowCfg;

constexpr uint32_t kKnownFlags = MOE_RENORM_TOPK | MOE_SAVE_ROW_STATS | MOE_WRITE_INV_PERM |
                                  MOE_SELECT_BIAS | MOE_P_MASKED | MOE_MULTI_KERNEL;
constexpr size_t kMaxLds = 160 * 1024;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const moe_route_params* p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 1 || p->E < 1 || p->k < 1 || p->n_micro < 1 || p->d < 0) return MOE_ERR_INVALID_ARG;
    if (p->k > p->E || p->T % p->n_micro != 0) return MOE_ERR_INVALID_ARG;
    if (p->E > MOE_ROUTE_MAX_E || p->k > MOE_ROUTE_MAX_K) return MOE_ERR_UNSUPPORTED;
    if (int64_t(p->T) * p->k > INT_MAX) return MOE_ERR_UNSUPPORTED;
    if (!std::isfinite(p->alpha) || !std::isfinite(p->capacity_factor)) return MOE_ERR_INVALID_ARG;
    if (p->capacity < -1) return MOE_ERR_INVALID_ARG;
    if (p->flags & ~kKnownFlags) return MOE_ERR_INVALID_ARG;
    if (p->d > 0 && !moe::gate_supported(p->T, p->d, p->E)) return MOE_ERR_UNSUPPORTED;
    const bool bias = (p->flags & MOE_SELECT_BIAS) != 0;
    const RowCfg c = moe::choose_rows(p->T, p->E, p->k, p->n_micro, bias, (p->flags & MOE_P_MASKED) != 0);
    if (c.G < 0 || moe::rows_lds_bytes(c, p->E, p->k, bias) > kMaxLds) return MOE_ERR_UNSUPPORTED;
    if (moe::scatter_lds_bytes(p->E, p->k, moe::scatter_waves(p->E, c.NW)) > kMaxLds) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

RowCfg cfg_of(const moe_route_params* p) {
    return moe::choose_rows(p->T, p->E, p->k, p->n_micro, (p->flags & MOE_SELECT_BIAS) != 0,
                            (p->flags & MOE_P_MASKED) != 0);
}

// Capacity of page mhpq.cn/news/998159 section 4.5: the per-expert share of
// a microbatch's Tm*k assignments, rounded up, times the capacity factor,
// rounded up.  The factor is the decimal the caller writes (1.1, 1.2, ...),
// which a double holds to within half an ulp; the product takes that error
// and its own rounding (together under 2^-52 relative), so a product within
// 2^-50 of an integer is that integer -- 1.1 * 50 is 55 although the double
// product is 55.000000000000007 -- and any other product is rounded up.  A
// factor with at most five decimal places and a product below 2^31 always
// keeps a fractional part of at least 1e-5, far outside that window.
int64_t capacity_of(const moe_route_params* p) {
    if (p->capacity >= 0) return p->capacity;
    if (!(p->capacity_factor > 0.0)) return -1;
    const int64_t Tm = p->T / p->n_micro;
    const int64_t per_expert = (Tm * p->k + p->E - 1) / p->E;
    const double x = p->capacity_factor * double(per_expert);
    const double r = std::nearbyint(x);
    const double c = (std::fabs(x - r) <= x * 0x1p-50) ? r : std::ceil(x);
    return c > double(INT_MAX) ? INT_MAX : int64_t(c);
}

size_t workspace_bytes(const moe_route_params* p, const RowCfg& c) {
    const size_t gate = p->d > 0 ? moe::gate_workspace_bytes(p->d, p->E) : 0;
    return moe::carve_workspace(nullptr, c, p->E, p->n_micro, gate).bytes;
}

// Device address of the scratch array on the current device, looked up once
// per device (the first moe_route_noalloc call there, with that device
// current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// One selection-bias step from counts [m,E] (the rule of moe_route_bias_update).
int bias_step(const moe_route_params* p, const int32_t* counts, float gamma, float* bias, hipStream_t st) {
    moe::BiasArgs b{counts, bias, p->E, p->n_micro, int64_t(p->T) * p->k, gamma};
    return moe::launch_bias_update(b, st) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

namespace moe {

hipError_t launch_route_rows(const RowCfg& c, const RowsArgs& a, hipStream_t st, const LaunchEvents* ev) {
    switch (c.S) {
        case 1: return launch_rows_s<1>(c, a, st, ev);
        case 2: return launch_rows_s<2>(c, a, st, ev);
        case 4: return launch_rows_s<4>(c, a, st, ev);
        case 8: return launch_rows_s<8>(c, a, st, ev);
        case 16: return launch_rows_s<16>(c, a, st, ev);
        case 32: return launch_rows_s<32>(c, a, st, ev);
        case 64: return launch_rows_s<64>(c, a, st, ev);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_route_backward(const RowCfg& c, const BackArgs& a, hipStream_t st) {
    switch (c.S) {
        case 1: return launch_backward_s<1>(c, a, st);
        case 2: return launch_backward_s<2>(c, a, st);
        case 4: return launch_backward_s<4>(c, a, st);
        case 8: return launch_backward_s<8>(c, a, st);
        case 16: return launch_backward_s<16>(c, a, st);
        case 32: return launch_backward_s<32>(c, a, st);
        case 64: return launch_backward_s<64>(c, a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe

extern "C" {

int moe_route_workspace_size(const moe_route_params* p, size_t* bytes) {
    const int rc = check_shape(p);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = workspace_bytes(p, cfg_of(p));
    return MOE_OK;
}

int moe_route_capacity(const moe_route_params* p, int32_t* capacity) {
    const int rc = check_shape(p);
    if (rc != MOE_OK) return rc;
    if (!capacity) return MOE_ERR_INVALID_ARG;
    *capacity = int32_t(capacity_of(p));
    return MOE_OK;
}

}  // extern "C"

namespace {

// The forward; with upd_bias, one selection-bias step from the call's counts
// follows (inside the scatter for one microbatch on the multi-kernel path,
// else by the update kernel after the forward).
int route_impl(const moe_route_params* p, const float* logits, const uint16_t* X, const uint16_t* Wg,
               const float* select_bias, const moe_route_out* out, void* workspace,
               size_t workspace_bytes_given, void* stream, float* upd_bias, float upd_gamma) {
    int rc = check_shape(p);
    if (rc != MOE_OK) return rc;
    if (!out) return MOE_ERR_INVALID_ARG;
    const bool gate = p->d > 0;
    if (gate) {
        if (!X || !Wg || !out->logits) return MOE_ERR_INVALID_ARG;
        if (!aligned(X, 16) || !aligned(Wg, 2) || !aligned(out->logits, 4)) return MOE_ERR_INVALID_ARG;
    } else {
        if (!logits || !aligned(logits, 4)) return MOE_ERR_INVALID_ARG;
    }
    if (!out->topk_idx || !out->topk_w || !out->counts || !out->offsets || !out->perm ||
        !out->dropped || !out->aux_loss || !out->cv || !out->max_over_mean)
        return MOE_ERR_INVALID_ARG;
    if ((p->flags & MOE_SAVE_ROW_STATS) && !out->row_stats) return MOE_ERR_INVALID_ARG;
    if ((p->flags & MOE_WRITE_INV_PERM) && !out->inv_perm) return MOE_ERR_INVALID_ARG;
    const bool bias = (p->flags & MOE_SELECT_BIAS) != 0;
    if (bias && (!select_bias || !aligned(select_bias, 4))) return MOE_ERR_INVALID_ARG;
    const void* fptrs[] = {out->topk_idx, out->topk_w, out->row_stats, out->counts, out->offsets,
                           out->perm, out->inv_perm, out->f, out->P, out->aux_loss, out->cv,
                           out->max_over_mean, out->extra_stats, out->status};
    for (const void* q : fptrs)
        if (q && !aligned(q, 4)) return MOE_ERR_INVALID_ARG;

    const RowCfg c = cfg_of(p);
    const size_t need = workspace_bytes(p, c);
    if (!workspace || workspace_bytes_given < need || !aligned(workspace, 256)) return MOE_ERR_WORKSPACE;
    const moe::Workspace ws = moe::carve_workspace(
        workspace, c, p->E, p->n_micro, gate ? moe::gate_workspace_bytes(p->d, p->E) : 0);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int Tm = p->T / p->n_micro;

    const float* L = logits;
    if (gate) {
        moe::GateArgs g{X, Wg, out->logits, p->T, p->d, p->E};
        if (moe::launch_gate_gemm(g, ws.Wt, st) != hipSuccess) return MOE_ERR_HIP;
        L = out->logits;
    }

    moe::RowsArgs ra{};
    ra.logits = L;
    ra.bias = bias ? select_bias : nullptr;
    ra.T = p->T; ra.E = p->E; ra.k = p->k; ra.Tm = Tm; ra.R = c.R; ra.bpm = c.bpm;
    ra.renorm = (p->flags & MOE_RENORM_TOPK) ? 1 : 0;
    ra.save_stats = (p->flags & MOE_SAVE_ROW_STATS) ? 1 : 0;
    ra.p_masked = (p->flags & MOE_P_MASKED) ? 1 : 0;
    ra.qcap = moe::rows_queue_cap(c);
    ra.topk_idx = out->topk_idx; ra.topk_w = out->topk_w; ra.row_stats = out->row_stats;
    ra.cnt_part = ws.cnt_part; ra.P_part = ws.P_part; ra.flag_part = ws.flag_part;
    ra.status = out->status;
    const bool timed = out->row_pass_events[0] && out->row_pass_events[1];
    const moe::LaunchEvents ev{static_cast<hipEvent_t>(out->row_pass_events[0]),
                               static_cast<hipEvent_t>(out->row_pass_events[1])};

    moe::ScatterArgs ca{};
    ca.n_micro = p->n_micro;
    ca.alpha = p->alpha;
    ca.p_masked = (p->flags & MOE_P_MASKED) ? 1 : 0;
    ca.counts = out->counts; ca.offsets = out->offsets; ca.f = out->f; ca.P = out->P;
    ca.aux = out->aux_loss; ca.cv = out->cv; ca.max_over_mean = out->max_over_mean;
    ca.extra = out->extra_stats;
    ca.T = p->T; ca.E = p->E; ca.k = p->k; ca.Tm = Tm;
    ca.capacity = int(capacity_of(p));
    ca.perm = out->perm;
    ca.inv_perm = (p->flags & MOE_WRITE_INV_PERM) ? out->inv_perm : nullptr;
    ca.dropped = out->dropped; ca.status = out->status;

    if (!(p->flags & MOE_MULTI_KERNEL) && moe::small_path_fits(Tm, p->E, p->k, p->n_micro)) {
        // small microbatches: the whole forward in one launch
        moe::SmallArgs sm{};
        sm.logits = L;
        sm.bias = ra.bias;
        sm.nb = moe::small_row_blocks(Tm);
        sm.renorm = ra.renorm; sm.save_stats = ra.save_stats;
        sm.topk_idx = out->topk_idx; sm.topk_w = out->topk_w; sm.row_stats = out->row_stats;
        sm.out = ca;
        if (moe::launch_route_small(sm, st, timed ? &ev : nullptr) != hipSuccess) return MOE_ERR_HIP;
        return upd_bias ? bias_step(p, out->counts, upd_gamma, upd_bias, st) : MOE_OK;
    }
    if (moe::launch_route_rows(c, ra, st, timed ? &ev : nullptr) != hipSuccess) return MOE_ERR_HIP;

    moe::ScanArgs sa{};
    sa.cnt_part = ws.cnt_part; sa.P_part = ws.P_part; sa.flag_part = ws.flag_part;
    sa.E = p->E; sa.k = p->k; sa.Tm = Tm; sa.bpm = c.bpm; sa.n_micro = p->n_micro; sa.B = c.B;
    sa.nsplit = c.nsplit;
    sa.colprefix = ws.colprefix; sa.split_tot = ws.split_tot; sa.split_P = ws.split_P;
    sa.status = out->status;
    // few row blocks per microbatch: the scatter sums their partials itself
    const int scat_nw = moe::scatter_waves(p->E, c.NW);
    const int fold_q = moe::scatter_fold_groups(p->E, p->k, c.bpm, scat_nw);
    if (fold_q == 0 && moe::launch_route_scan(c, sa, st) != hipSuccess) return MOE_ERR_HIP;

    ca.topk_idx = out->topk_idx; ca.colprefix = ws.colprefix; ca.split_tot = ws.split_tot;
    ca.split_P = ws.split_P;
    ca.cnt_part = ws.cnt_part; ca.P_part = ws.P_part; ca.flag_part = ws.flag_part;
    ca.fold_q = fold_q; ca.B = c.B; ca.nw = scat_nw;
    // few row blocks: the statistics get workgroups of their own, so that no
    // block adds them to its share of the permutation -- when the row blocks
    // and those workgroups fit the chip at once, or when two eight-wave
    // scatter blocks share a compute unit and the grid stays within two a
    // compute unit (65536 tokens, E=64 top-2: 19.0 -> 18.4 us a call)
    const bool fit_one = c.B + p->n_micro <= moe::kAssumedCUs;
    const bool fit_two = scat_nw == 8 && c.B + p->n_micro <= 2 * moe::kAssumedCUs &&
                         moe::scatter_lds_bytes(p->E, p->k, 8) <= 64 * 1024;
    ca.stats_sep = (fit_one || fit_two) ? 1 : 0;
    ca.bpm = c.bpm; ca.nsplit = c.nsplit;
    ca.rows_per_wave = moe::scatter_rows_per_wave(p->E, p->k, scat_nw);
    ca.vec_idx = (p->k % 4 == 0 && aligned(out->topk_idx, 16)) ? 1 : 0;
    const bool fused_step = upd_bias && p->n_micro == 1;
    ca.upd_bias = fused_step ? upd_bias : nullptr;
    ca.upd_gamma = upd_gamma;
    if (moe::launch_route_scatter(c, ca, st) != hipSuccess) return MOE_ERR_HIP;
    return (upd_bias && !fused_step) ? bias_step(p, out->counts, upd_gamma, upd_bias, st) : MOE_OK;
}

}  // namespace

extern "C" {

int moe_route(const moe_route_params* p, const float* logits, const uint16_t* X,
              const uint16_t* Wg, const float* select_bias, const moe_route_out* out,
              void* workspace, size_t workspace_bytes_given, void* stream) {
    return route_impl(p, logits, X, Wg, select_bias, out, workspace, workspace_bytes_given, stream, nullptr, 0.f);
}

int moe_route_with_bias_update(const moe_route_params* p, const float* logits, const uint16_t* X,
                               const uint16_t* Wg, float* select_bias, float gamma, const moe_route_out* out,
                               void* workspace, size_t workspace_bytes_given, void* stream) {
    if (!p || !(p->flags & MOE_SELECT_BIAS)) return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(gamma) || gamma < 0.f) return MOE_ERR_INVALID_ARG;
    return route_impl(p, logits, X, Wg, select_bias, out, workspace, workspace_bytes_given, stream,
                      select_bias, gamma);
}

int moe_route_noalloc(const moe_route_params* p, const float* logits, const uint16_t* X,
                      const uint16_t* Wg, const float* select_bias, const moe_route_out* out,
                      void* stream) {
    const int rc = check_shape(p);
    if (rc != MOE_OK) return rc;
    if (workspace_bytes(p, cfg_of(p)) > size_t(MOE_ROUTE_SCRATCH_BYTES)) return MOE_ERR_SCRATCH;
    void* ws = nullptr;
    const int sc = scratch_of_current_device(&ws);
    if (sc != MOE_OK) return sc;
    return moe_route(p, logits, X, Wg, select_bias, out, ws, size_t(MOE_ROUTE_SCRATCH_BYTES), stream);
}

int moe_route_backward(const moe_route_params* p, const float* logits, const float* row_stats,
                       const int32_t* counts, const float* d_aux, const int32_t* topk_idx,
                       const float* d_topk_w, float* dlogits, void* stream) {
    if (!p) return MOE_ERR_INVALID_ARG;
    moe_route_params q = *p;
    q.d = 0;  // the backward reads logits whatever produced them
    const int rc = check_shape(&q);
    if (rc != MOE_OK) return rc;
    if (!logits || !counts || !dlogits) return MOE_ERR_INVALID_ARG;
    const bool masked = (q.flags & MOE_P_MASKED) != 0;
    if ((masked || d_topk_w) && !topk_idx) return MOE_ERR_INVALID_ARG;
    const void* ptrs[] = {logits, row_stats, counts, d_aux, topk_idx, d_topk_w, dlogits};
    for (const void* x : ptrs)
        if (x && !aligned(x, 4)) return MOE_ERR_INVALID_ARG;
    const RowCfg c = moe::choose_rows(q.T, q.E, q.k, q.n_micro);
    if ((masked || d_topk_w) && moe::backward_lds_bytes(c, q.E) > kMaxLds) return MOE_ERR_UNSUPPORTED;
    moe::BackArgs b{};
    b.logits = logits; b.row_stats = row_stats; b.counts = counts; b.d_aux = d_aux; b.dlogits = dlogits;
    b.topk_idx = topk_idx; b.d_topk_w = d_topk_w;
    b.T = q.T; b.E = q.E; b.k = q.k; b.Tm = q.T / q.n_micro; b.R = c.R; b.bpm = c.bpm;
    b.alpha = q.alpha;
    b.p_masked = masked ? 1 : 0;
    b.renorm = (q.flags & MOE_RENORM_TOPK) ? 1 : 0;
    if (moe::launch_route_backward(c, b, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_route_bias_update(const moe_route_params* p, const int32_t* counts, float gamma,
                          float* bias, void* stream) {
    if (!p) return MOE_ERR_INVALID_ARG;
    moe_route_params q = *p;
    q.d = 0;
    q.flags = 0;
    const int rc = check_shape(&q);
    if (rc != MOE_OK) return rc;
    if (!counts || !bias || !aligned(counts, 4) || !aligned(bias, 4)) return MOE_ERR_INVALID_ARG;
    if (!std::isfinite(gamma) || gamma < 0.f) return MOE_ERR_INVALID_ARG;
    moe::BiasArgs b{counts, bias, q.E, q.n_micro, int64_t(q.T) * q.k, gamma};
    if (moe::launch_bias_update(b, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

static int check_gate_backward(const moe_route_params* p) {
    if (!p || p->T < 1 || p->E < 1 || p->d < 1) return MOE_ERR_INVALID_ARG;
    if (!moe::gate_supported(p->T, p->d, p->E)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int moe_gate_backward_workspace_size(const moe_route_params* p, size_t* bytes) {
    const int rc = check_gate_backward(p);
    if (rc != MOE_OK) return rc;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = moe::gate_backward_workspace_bytes(p->T, p->d, p->E);
    return MOE_OK;
}

int moe_gate_backward(const moe_route_params* p, const uint16_t* X, const uint16_t* Wg,
                      const float* dlogits, uint16_t* dX, float* dWg, void* workspace,
                      size_t workspace_bytes_given, void* stream) {
    const int rc = check_gate_backward(p);
    if (rc != MOE_OK) return rc;
    if (!X || !Wg || !dlogits || (!dX && !dWg)) return MOE_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Wg, 2) || !aligned(dlogits, 4) || (dX && !aligned(dX, 16)) ||
        (dWg && !aligned(dWg, 4)))
        return MOE_ERR_INVALID_ARG;
    if (dWg) {
        const size_t need = moe::gate_backward_workspace_bytes(p->T, p->d, p->E);
        if (!workspace || workspace_bytes_given < need || !aligned(workspace, 256)) return MOE_ERR_WORKSPACE;
    }
    moe::GateBackArgs g{X, Wg, dlogits, dX, dWg, static_cast<float*>(workspace), p->T, p->d, p->E};
    if (moe::launch_gate_backward(g, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_eplb_plan(int32_t E, int32_t num_phys, int32_t num_packs, const int32_t* weight,
                  int32_t* phy2log, int32_t* phy_rank, int32_t* logcnt, int32_t* pack, int32_t* slot,
                  double* pack_load, void* stream) {
    if (E < 1 || num_phys < E || num_packs < 1 || num_phys % num_packs != 0) return MOE_ERR_INVALID_ARG;
    if (E > MOE_ROUTE_MAX_E || num_phys > MOE_EPLB_MAX_PHYS || num_packs > MOE_EPLB_MAX_PACKS)
        return MOE_ERR_UNSUPPORTED;
    const void* ptrs[] = {weight, phy2log, phy_rank, logcnt, pack, slot};
    for (const void* q : ptrs)
        if (!q || !aligned(q, 4)) return MOE_ERR_INVALID_ARG;
    if (!pack_load || !aligned(pack_load, 8)) return MOE_ERR_INVALID_ARG;
    moe::EplbArgs e{weight, phy2log, phy_rank, logcnt, pack, slot, pack_load, E, num_phys, num_packs};
    if (moe::launch_eplb(e, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_sinkhorn_plan(int32_t R, const double* supply, const double* demand, const double* cost,
                      double eps, int32_t iters, double* u, double* v, double* T, void* stream) {
    if (R < 1 || iters < 0 || !(eps > 0.0) || !std::isfinite(eps)) return MOE_ERR_INVALID_ARG;
    if (R > MOE_SINKHORN_MAX_R || iters > MOE_SINKHORN_MAX_ITERS) return MOE_ERR_UNSUPPORTED;
    const void* ptrs[] = {supply, demand, cost, u, v, T};
    for (const void* q : ptrs)
        if (!q || !aligned(q, 8)) return MOE_ERR_INVALID_ARG;
    moe::SinkhornArgs k{supply, demand, cost, u, v, T, eps, R, iters};
    if (moe::launch_sinkhorn(k, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

const char* moe_route_strerror(int code) {
    switch (code) {
        case MOE_OK: return "success";
        case MOE_ERR_INVALID_ARG: return "invalid argument (NULL pointer, misaligned pointer, bad shape or value)";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape (E, k, T*k or gate dimensions beyond the limits)";
        case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than moe_route_workspace_size()";
        case MOE_ERR_HIP: return "a HIP kernel launch failed";
        case MOE_ERR_SCRATCH:
            return "moe_route_noalloc: the shape needs more workspace than MOE_ROUTE_SCRATCH_BYTES (32 MiB)";
        default: return "unknown moe_route error code";
    }
}

}  // extern "C"
