// api.cpp -- the C ABI: argument checks, the planner and the launch sequence.
//
// Entry points and their contract are declared in include/conv2d_grad_input.h.
// Shape fields mirror the Params block of meganeura conv2d_grad_input_gemm.wgsl
// and the options of doppler conv2d_backward.d.ts (Conv2DBackwardOptions).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

#include "conv2d_grad_input.h"
#include "conv2d_grad_input_testing.h"
#include "gi_common.h"
#include "gi_launch.h"
#include "fwd_common.h"
#include "gw_common.h"
#include "half_launch.h"
#include "api_internal.h"

namespace {

using gi::GemmArgs;
using gi::Phase;

// Test and diagnostic hooks (conv2d_grad_input_testing.h): thread-local, so a
// setting changes only the plans of the thread that made it.
thread_local int g_variant = CONV2D_GI_VARIANT_AUTO;
// Forced halo tile: NB pixel blocks, TR x TC phase-grid pixels; 0 = planner.
thread_local int g_tile_nb = 0, g_tile_tr = 0, g_tile_tc = 0, g_tile_stages = 0;
thread_local int g_halo_split = 0;
thread_local int g_halo_fusion = 0;  // 0 planner, 1 phase at a time, 2 fused
thread_local int g_gw_variant = 0;   // grad_weight: 0 planner, 1 4-byte loads, 2 16-byte loads
thread_local int g_fwd_variant = 0;  // forward: 0 planner, 1 grad_input kernels, 2 generic
thread_local int g_gw_rows = 0;      // grad_weight, 16-byte loads: forced rows per group (0 planner)
thread_local int g_gw_stages = 0;    // ... and LDS stages (0 planner)
thread_local int g_gw_slices = 0;    // ... and most slices (0 planner)
thread_local char g_last_hip[256] = "";
thread_local hipEvent_t g_prof_begin = nullptr, g_prof_end = nullptr;

// Scratch (the reordered weight) cached per (device, stream): allocated
// stream-ordered on first use, grown when a call needs more, reused by later
// calls on the same stream (stream order keeps them apart), released by
// conv2d_gi_release_workspaces.  The lock is held while a call enqueues; it is
// recursive so that an entry point that fills one slot and then runs another
// path reading it keeps the lock across both.
struct Workspace {
    void *ptr = nullptr;
    size_t bytes = 0;
};
std::recursive_mutex g_ws_mu;
// Scratch per (device, stream, slot): slot 0 serves every kernel's own
// scratch, slot 1 a reordered operand that a later call in the same entry
// point reads (the forward's reversed weight).
std::map<std::tuple<int, hipStream_t, int>, Workspace> g_ws;

hipError_t workspace_for(int dev, hipStream_t s, size_t bytes, void **out, int slot = 0) {
    Workspace &w = g_ws[std::make_tuple(dev, s, slot)];
    if (w.bytes < bytes) {
        if (w.ptr) {
            hipError_t e = hipFreeAsync(w.ptr, s);
            w.ptr = nullptr;
            w.bytes = 0;
            if (e != hipSuccess) return e;
        }
        hipError_t e = hipMallocAsync(&w.ptr, bytes, s);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return e;
        }
        w.bytes = bytes;
    }
    *out = w.ptr;
    return hipSuccess;
}

int fail_hip(hipError_t e) {
    std::snprintf(g_last_hip, sizeof(g_last_hip), "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return CONV2D_GI_EHIP;
}

int64_t floordiv(int64_t a, int64_t b) {  // b > 0
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// Shape checks shared by every entry point (host only, no HIP call).
int validate(const conv2d_gi_params *p) {
    if (!p) return CONV2D_GI_EINVAL;
    // Every size is at least 1: the doppler wrappers throw on a missing or
    // zero size, so a valid call always has elements in every tensor.
    if (p->N < 1 || p->Ci < 1 || p->Co < 1) return CONV2D_GI_EINVAL;
    if (p->H < 1 || p->W < 1 || p->kH < 1 || p->kW < 1 || p->stride < 1) return CONV2D_GI_EINVAL;
    if (p->pad_h < 0 || p->pad_w < 0) return CONV2D_GI_EINVAL;
    const int64_t oH = floordiv((int64_t)p->H + 2LL * p->pad_h - p->kH, p->stride) + 1;
    const int64_t oW = floordiv((int64_t)p->W + 2LL * p->pad_w - p->kW, p->stride) + 1;
    if (oH < 1 || oW < 1) return CONV2D_GI_EINVAL;
    if (p->oH != oH || p->oW != oW) return CONV2D_GI_EINVAL;
    // Index width: per-image planes, the weight and the folded pixel axes
    // (input and output side) are addressed with 32-bit offsets inside the
    // kernels; batch offsets are 64-bit.
    const int64_t lim = INT32_MAX;
    if ((int64_t)p->Ci * p->H * p->W > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->Co * oH * oW > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->Co * p->Ci * p->kH * p->kW > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->N * p->H * p->W > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->N * oH * oW > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((p->Ci + gi::kGenericBM - 1) / gi::kGenericBM > 65535) return CONV2D_GI_EUNSUPPORTED;
    return CONV2D_GI_OK;
}

// Residue classes of the stride that own at least one input pixel.
std::vector<Phase> make_phases(const conv2d_gi_params &p) {
    std::vector<Phase> out;
    const int s = p.stride;
    for (int rh = 0; rh < s && rh < p.H; ++rh) {
        for (int rw = 0; rw < s && rw < p.W; ++rw) {
            Phase ph{};
            ph.rho_h = rh;
            ph.rho_w = rw;
            ph.q_h = (rh + p.pad_h) / s;
            ph.q_w = (rw + p.pad_w) / s;
            ph.r_h = (rh + p.pad_h) % s;
            ph.r_w = (rw + p.pad_w) % s;
            ph.J_h = ph.r_h < p.kH ? (p.kH - ph.r_h + s - 1) / s : 0;
            ph.J_w = ph.r_w < p.kW ? (p.kW - ph.r_w + s - 1) / s : 0;
            ph.Ha = (p.H - rh + s - 1) / s;
            ph.Wb = (p.W - rw + s - 1) / s;
            out.push_back(ph);
        }
    }
    return out;
}

struct Launch {
    GemmArgs args;
    int tiles_x;
};

// A halo-kernel plan (fp32): one launch over every phase.
struct HaloPlan {
    gi::HaloArgs args{};
    int nb = 0, cfg = -1, bl = 0, tiles = 0, ci_tiles = 0;
    size_t lds = 0;
    double cost = 0.0;
    int64_t ws_floats = 0;  // weight image
    int fused = 0;           // all phases per chunk over one shared halo
};

// A bf16 halo-kernel plan (stride 1): two prologues and one launch.
struct HaloBf16Plan {
    gi::HaloBf16Args args{};
    int cfg = -1, tiles = 0, ci_tiles = 0;
    size_t lds = 0;
    size_t gp_bytes = 0, wk_bytes = 0;  // workspace: padded grad_out, then weight fragments
    double cost = 0.0;
};

// A whole-image 16-bit plan (stride 1): a weight prologue and one launch.
struct Img16Plan {
    gi::Img16Args args{};
    int cfg = -1;
    size_t lds = 0;
    size_t wk_bytes = 0;   // workspace: the weight fragment image
    int wtiles = 0;        // its 64-channel ci tiles
};

// A small-Ci plan (fp32, Ci <= 4): one prologue and one launch.
struct StemPlan {
    gi::StemArgs args{};
    size_t ws_bytes = 0;
};

struct Col2imPlan {
    gi::Col2imArgs args{};
    size_t lds = 0;
};

struct Plan {
    int variant = CONV2D_GI_VARIANT_GENERIC;
    bool bf16 = false;
    size_t ws_bytes = 0;  // reordered weight
    std::vector<Launch> launches;  // generic
    HaloPlan halo;                 // halo, fp32
    HaloBf16Plan hb;               // halo, bf16
    bool img16 = false;            // 16-bit inputs on the whole-image kernel
    Img16Plan im;
    StemPlan stem;                 // small Ci, fp32
    Col2imPlan c2i;                // few columns, fp32
};

constexpr int kCUs = 256;               // MI355X compute units
constexpr size_t kLdsBytes = 160 * 1024;


// Smallest p >= v with p % m == r (0 <= r < m).
int round_to_residue(int v, int m, int r) {
    int p = v + ((r - v % m) % m + m) % m;
    return p;
}

// Halo plan for fp32: choose the pixel tile (TR x TC of the phase grid, at
// most NB*16 pixels) that minimises the work of the busiest compute unit,
// ceil(work-groups / CUs) x (MFMA cycles of one work-group + staging + a
// fixed per-work-group cost), among the instantiated kernels that fit.
bool plan_halo(const conv2d_gi_params &p, const std::vector<Phase> &phases, HaloPlan &out) {
    if (phases.empty() || (int)phases.size() > gi::kMaxPhasesPerLaunch) return false;
    // Buffer offsets inside the kernel are 32-bit byte offsets.
    const int64_t lim = 0x7fff0000LL;
    if ((int64_t)p.N * p.Co * p.oH * p.oW * 4 > lim) return false;
    if ((int64_t)p.N * p.Ci * p.H * p.W * 4 > lim) return false;
    int maxT = 0, maxJh = 0, maxJw = 0, maxHa = 0, maxWb = 0;
    bool fold = true;
    const int nchunks = (p.Co + gi::kHaloBC - 1) / gi::kHaloBC;
    int64_t kall = 0;  // sum over phases of padded Co x taps
    int64_t w_ci_stride = 0;
    unsigned tmask = 0;
    for (const Phase &ph : phases) {
        const int T = ph.J_h * ph.J_w;
        if (T > 0) {
            // A tap count no instance serves (0: past the mask's range) rules
            // the halo kernels out.
            const unsigned bit = gi::halo_f32_tbit(T);
            if (bit == 0) return false;
            tmask |= bit;
        }
        maxT = std::max(maxT, T);
        maxJh = std::max(maxJh, ph.J_h);
        maxJw = std::max(maxJw, ph.J_w);
        maxHa = std::max(maxHa, ph.Ha);
        maxWb = std::max(maxWb, ph.Wb);
        if (ph.J_h > 1) fold = false;
        kall += (int64_t)nchunks * gi::kHaloBC * T;
        w_ci_stride += (int64_t)nchunks * T * 512;
    }
    // The kernel-width tap count shared by every phase with taps (0 if not).
    int jw_common = -1;
    for (const Phase &ph : phases) {
        if (ph.J_h * ph.J_w == 0) continue;
        jw_common = jw_common < 0 || jw_common == ph.J_w ? ph.J_w : 0;
    }
    if (jw_common < 0) jw_common = 0;
    const int ci_tiles = (p.Ci + gi::kHaloCT - 1) / gi::kHaloCT;
    if (w_ci_stride * ci_tiles * 4 > lim || maxT == 0) return false;
    // Fused launches (every phase per chunk over one halo): four phases with
    // tap grids of at most 2 x 2.  The shared halo starts at the smallest
    // phase origin q - (J - 1) and reaches TR + ur rows, TC + uc columns.
    int Tall = 0, org_h = INT32_MAX, org_w = INT32_MAX, ur = 0, uc = 0;
    bool fusable = phases.size() == 4 && !fold && g_halo_fusion != 1;
    for (const Phase &ph : phases) {
        Tall += ph.J_h * ph.J_w;
        if (ph.J_h > 2 || ph.J_w > 2) fusable = false;
        if (ph.J_h * ph.J_w == 0) continue;
        org_h = std::min(org_h, ph.q_h - (ph.J_h - 1));
        org_w = std::min(org_w, ph.q_w - (ph.J_w - 1));
    }
    if (Tall == 0 || Tall > 12) fusable = false;
    if (fusable)
        for (const Phase &ph : phases) {
            if (ph.J_h * ph.J_w == 0) continue;
            ur = std::max(ur, ph.q_h - (ph.J_h - 1) - org_h + ph.J_h - 1);
            uc = std::max(uc, ph.q_w - (ph.J_w - 1) - org_w + ph.J_w - 1);
        }
    const int fz_lo = g_halo_fusion == 2 ? 1 : 0;
    static const int kNB[] = {4, 8, 13};
    const int f_nb = g_tile_nb, f_tr = g_tile_tr, f_tc = g_tile_tc;
    const bool forced = f_nb > 0;
    bool found = false;
    for (int nb : kNB) {
        if (forced && nb != f_nb) continue;
        const int maxpx = nb * 16;
        for (int cdiv = 1; cdiv <= (forced ? 1 : 8); ++cdiv) {
            const int TC = forced ? f_tc : (maxWb + cdiv - 1) / cdiv;
            if (!forced && cdiv > 1 && TC == (maxWb + cdiv - 2) / (cdiv - 1)) continue;
            if (TC > maxpx) continue;
            const int rows_total = fold ? p.N * maxHa : maxHa;
            for (int TR = forced ? f_tr : std::min(maxpx / TC, rows_total); TR >= 1; --TR) {
                if (forced && (TR != f_tr || TR * TC > maxpx)) break;
                if (!forced && nb > 4 && TR * TC <= (nb == 8 ? 4 : 8) * 16) break;
                for (int fz = fz_lo; fz <= (fusable ? 1 : 0); ++fz) {
                const int HR = fz ? TR + ur : TR + maxJh - 1;
                const int HC = fz ? TC + uc : TC + maxJw - 1;
                // Halo row pitch: the padded one (= TC mod 16) puts the 16
                // pixels of a block (which may wrap to the next tile row) at
                // positions distinct mod 16, so the fragment reads of a
                // half-wave are conflict-free; it costs LDS and staging.
                for (int padded = 1; padded >= 0; --padded) {
                const int HP = padded ? round_to_residue(HC, 16, TC % 16) : HC;
                if (padded && HP == HC) continue;
                // Halo positions are staged in groups of 32, the groups dealt
                // round-robin to the 4 waves; the co-pair pitch sits 16 float2
                // off a multiple of 32 so the co-pair rows of a fragment read
                // fall on disjoint banks.
                const int groups = (HR * HP + 31) / 32;
                // ks thread groups split each work-group's output channels
                // (phase at a time) or its phases (fused: always two, sharing
                // every stage).
                for (int ks = fz ? 2 : 1; ks <= 2; ++ks) {
                const int f_ks = g_halo_split;
                if (!fz && f_ks > 0 && ks != f_ks) continue;
                const int bl = fz ? (groups + 4 * ks - 1) / (4 * ks) : (groups + 3) / 4;
                const int cfg = gi::halo_f32_config(nb, tmask, bl, HP, jw_common, ks, fz ? 4 : 0);
                if (cfg < 0) continue;
                const int HPc = round_to_residue(groups * 32, 32, 16);
                const int cps = gi::halo_f32_cps(cfg);
                // A fused stage holds the weights of every phase's taps.
                const int stage_taps = fz ? Tall : maxT;
                // Three pipeline stages when two work-groups (or two thread
                // groups) still fit a CU, or when one is all that fits anyway.
                const size_t budget = kLdsBytes / 2;
                int stages = 3;
                size_t lds = gi::halo_f32_lds_bytes(stage_taps, HPc, 3, cps);
                if (lds > budget) {
                    stages = 2;
                    lds = gi::halo_f32_lds_bytes(stage_taps, HPc, 2, cps);
                    if (lds > budget && ks == 1 &&
                        gi::halo_f32_lds_bytes(stage_taps, HPc, 3, cps) <= kLdsBytes) {
                        stages = 3;
                        lds = gi::halo_f32_lds_bytes(stage_taps, HPc, 3, cps);
                    }
                }
                if (forced && g_tile_stages > 0) {
                    stages = g_tile_stages;
                    lds = gi::halo_f32_lds_bytes(stage_taps, HPc, stages, cps);
                }
                // A split work-group holds every group's stages, and its
                // accumulators once, for the hand-over (fused groups share
                // the stages and hand nothing over).
                if (!fz) lds = std::max(lds * ks, ks > 1 ? (size_t)nb * 256 * 16 : (size_t)0);
                if (lds > kLdsBytes) continue;
                const int64_t row_tiles = (rows_total + TR - 1) / TR;
                const int64_t col_tiles = (maxWb + TC - 1) / TC;
                const int64_t tiles = row_tiles * col_tiles * (fold ? 1 : p.N);
                if (tiles > INT32_MAX) continue;
                const int64_t wgs = tiles * ci_tiles;
                // Busiest CU: ceil(work-groups / CUs) work-groups.  Measured
                // efficiency of the instantiations: more pixel blocks per wave
                // amortise more per-tap and per-chunk overhead, a lone
                // work-group per CU hides less latency, and conflict-free
                // fragment reads with compile-time tap offsets save time.
                const int64_t per_cu = (wgs + kCUs - 1) / kCUs;
                const double eff_nb = nb >= 13 ? 1.0 : nb >= 8 ? 0.85 : 0.75;
                // One wave per SIMD (a lone unsplit work-group per CU) hides
                // less latency.
                const double eff_occ = per_cu >= 2 || ks > 1 ? 1.0 : 0.9;
                const bool conflict_free = (HP - TC) % 16 == 0 || TC % 16 == 0;
                const double eff_pitch = (gi::halo_f32_fixed_pitch(cfg) ? 1.05 : 1.0) *
                                         (conflict_free ? 1.03 : 1.0);
                // 16x16x4 MFMA: 32 cycles per 16 pixels x 4 k; plus halo staging.
                // Halo staging: once per chunk when fused, else once per phase.
                const double per_wg = 8.0 * nb * kall +
                                      (double)nchunks * (fz ? 1 : phases.size()) * HR * HP * 2.0 +
                                      4000.0 + (ks > 1 ? 1500.0 * phases.size() : 0.0);
                // Among equal critical paths, fewer work-groups do less total work.
                const double cost = (double)per_cu * per_wg / (eff_nb * eff_occ * eff_pitch) +
                                    0.05 * (double)wgs * per_wg / kCUs;
                if (!found || cost < out.cost) {
                    found = true;
                    out = HaloPlan{};
                    out.cost = cost;
                    out.nb = nb;
                    out.cfg = cfg;
                    out.bl = bl;
                    out.tiles = (int)tiles;
                    out.ci_tiles = ci_tiles;
                    out.lds = lds;
                    out.fused = fz;
                    gi::HaloArgs &a = out.args;
                    a.TR = TR;
                    a.TC = TC;
                    a.row_tiles = (int)row_tiles;
                    a.col_tiles = (int)col_tiles;
                    a.HP = HP;
                    a.HPc = HPc;
                    a.stages = stages;
                    a.HR = HR;
                    a.HC = HC;
                }
                }
                }
                }
            }
        }
    }
    if (!found) return false;
    gi::HaloArgs &a = out.args;
    a.g_bytes = (uint32_t)((int64_t)p.N * p.Co * p.oH * p.oW * 4);
    a.d_bytes = (uint32_t)((int64_t)p.N * p.Ci * p.H * p.W * 4);
    a.w_bytes = (uint32_t)(w_ci_stride * ci_tiles * 4);
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.oH = p.oH;
    a.oW = p.oW;
    a.stride = p.stride;
    a.fold = fold ? 1 : 0;
    a.nchunks = nchunks;
    a.maxT = maxT;
    a.w_ci_stride = (int)w_ci_stride;
    a.ci_tiles = ci_tiles;
    a.nphases = (int)phases.size();
    int64_t woff = 0;
    for (size_t i = 0; i < phases.size(); ++i) {
        const Phase &ph = phases[i];
        gi::HaloPhase &h = a.ph[i];
        h.rho_h = ph.rho_h;
        h.rho_w = ph.rho_w;
        h.q_h = ph.q_h;
        h.q_w = ph.q_w;
        h.r_h = ph.r_h;
        h.r_w = ph.r_w;
        h.J_h = ph.J_h;
        h.J_w = ph.J_w;
        h.Ha = ph.Ha;
        h.Wb = ph.Wb;
        h.woff = (int)woff;
        woff += (int64_t)nchunks * ph.J_h * ph.J_w * 512;
    }
    out.ws_floats = w_ci_stride * ci_tiles;
    a.fused = out.fused;
    if (out.fused) {
        a.Tall = Tall;
        a.org_h = org_h;
        a.org_w = org_w;
        int tb = 0;
        for (size_t i = 0; i < phases.size(); ++i) {
            const Phase &ph = phases[i];
            gi::HaloPhase &h = a.ph[i];
            h.tb = tb;
            tb += ph.J_h * ph.J_w;
            h.dr = ph.J_h * ph.J_w ? ph.q_h - (ph.J_h - 1) - org_h : 0;
            h.dc = ph.J_h * ph.J_w ? ph.q_w - (ph.J_w - 1) - org_w : 0;
        }
        // Two thread groups: the phases sorted by taps, the largest with the
        // smallest in one group and the middle two in the other, so the
        // groups' tap totals are close.
        int order[4] = {0, 1, 2, 3};
        std::stable_sort(order, order + 4, [&](int x, int y) {
            return phases[x].J_h * phases[x].J_w > phases[y].J_h * phases[y].J_w;
        });
        std::memset(a.gph, -1, sizeof(a.gph));
        a.gph[0][0] = (int8_t)order[0];
        a.gph[0][1] = (int8_t)order[3];
        a.gph[1][0] = (int8_t)order[1];
        a.gph[1][1] = (int8_t)order[2];
    }
    if (!out.fused) {
        std::memset(a.gph, -1, sizeof(a.gph));
    }
    return true;
}

// bf16 halo plan (stride 1, tap counts the kernel is built for): choose the
// TR x TC pixel tile (at most 2*NBW*16 pixels, halo at most 256 positions)
// that minimises ceil(work-groups / CUs) x per-work-group MFMA cycles.
bool plan_halo_bf16(const conv2d_gi_params &p, HaloBf16Plan &out) {
    if (p.stride != 1 || p.Ci < 16) return false;
    const int T = p.kH * p.kW;
    const int nchunks = (p.Co + 31) / 32;
    const int Cop = nchunks * 32;
    const int YP = p.H + p.kH - 1, XP = p.W + p.kW - 1;
    const int ci_tiles = (p.Ci + 63) / 64;
    const int64_t lim = 0x7fff0000LL;
    const int64_t gp_bytes = (int64_t)p.N * YP * XP * Cop * 2;
    const int64_t wk_bytes = (int64_t)ci_tiles * 64 * Cop * T * 2;
    if (gp_bytes > lim || wk_bytes > lim || (int64_t)p.N * p.Ci * p.H * p.W * 4 > lim)
        return false;
    static const int kNBW[] = {4, 7};
    const int f_nb = g_tile_nb, f_tr = g_tile_tr, f_tc = g_tile_tc;
    const bool forced = f_nb > 0;
    bool found = false;
    for (int nbw : kNBW) {
        if (forced && nbw != f_nb) continue;
        const int maxpx = 2 * nbw * 16;
        for (int cdiv = 1; cdiv <= (forced ? 1 : 8); ++cdiv) {
            const int TC = forced ? f_tc : (p.W + cdiv - 1) / cdiv;
            if (!forced && cdiv > 1 && TC == (p.W + cdiv - 2) / (cdiv - 1)) continue;
            if (TC > maxpx) continue;
            for (int TR = forced ? f_tr : std::min(maxpx / TC, p.H); TR >= 1; --TR) {
                if (forced && (TR != f_tr || TR * TC > maxpx)) break;
                const int HR = TR + p.kH - 1, HC = TC + p.kW - 1;
                // Row pitch: holds a halo row, and = TC mod 16.
                const int HP = round_to_residue(HC, 16, TC % 16);
                const int nql = (HR * HP + 63) / 64;
                if (nql > gi::kHaloBf16Loads) continue;
                const int cfg = gi::halo_bf16_config(nbw, p.kH, p.kW, HP);
                if (cfg < 0) continue;
                const int64_t tiles = (int64_t)((p.H + TR - 1) / TR) * ((p.W + TC - 1) / TC) * p.N;
                if (tiles > INT32_MAX) continue;
                const int64_t wgs = tiles * ci_tiles;
                const double rounds = (double)((wgs + kCUs - 1) / kCUs);
                // 16x16x32 MFMA, 16 cycles: 2 ci blocks x nbw pixel blocks per wave per k step.
                const double per_wg = 16.0 * 2 * nbw * (double)nchunks * T + 3000.0;
                const double cost = rounds * per_wg + 0.05 * (double)wgs * per_wg / kCUs;
                if (!found || cost < out.cost) {
                    found = true;
                    out = HaloBf16Plan{};
                    out.cost = cost;
                    out.cfg = cfg;
                    out.tiles = (int)tiles;
                    out.ci_tiles = ci_tiles;
                    gi::HaloBf16Args &a = out.args;
                    a.TR = TR;
                    a.TC = TC;
                    a.HR = HR;
                    a.HC = HC;
                    a.row_tiles = (p.H + TR - 1) / TR;
                    a.col_tiles = (p.W + TC - 1) / TC;
                    a.HP = HP;
                    a.nql = nql;
                    a.PS = nql * 1024;
                }
            }
        }
    }
    if (!found) return false;
    gi::HaloBf16Args &a = out.args;
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.kH = p.kH;
    a.kW = p.kW;
    a.YP = YP;
    a.XP = XP;
    a.Cop = Cop;
    a.nchunks = nchunks;
    a.ci_tiles = ci_tiles;
    a.gp_bytes = (uint32_t)gp_bytes;
    a.wk_bytes = (uint32_t)wk_bytes;
    a.d_bytes = (uint32_t)((int64_t)p.N * p.Ci * p.H * p.W * 4);
    out.lds = (size_t)2 * 4 * a.PS + 1024;  // 2 stages of 4 planes + a scratch kilobyte
    out.gp_bytes = (size_t)(gp_bytes + 255) / 256 * 256;
    out.wk_bytes = (size_t)wk_bytes;
    return true;
}

// Whole-image 16-bit plan (stride 1): one work-group per (image, 128 input
// channels), every pixel of the image in the wave's 16-pixel blocks.  Needs
// an instance for the pixel blocks, taps, kernel width and halo pitch, a
// grad_out plane of whole 4-pixel quads of which 8 planes fit a wave's 4 KB
// landing area, an image of whole 4-pixel quads, and 32-bit byte offsets.
bool plan_img16(const conv2d_gi_params &p, Img16Plan &out) {
    if (p.stride != 1) return false;
    const int HW = p.H * p.W, oHW = p.oH * p.oW;
    // Each wave copies 8 grad_out planes (plus up to 8 bytes of alignment)
    // into a 4 KB landing area, and its lanes take one 4-pixel quad each;
    // the epilogue stores whole 4-pixel quads of the image.
    if (oHW % 4 != 0 || 8 + 16 * oHW > 4096 || HW % 4 != 0) return false;
    const int HR = p.H + p.kH - 1, HC = p.W + p.kW - 1;
    const int HP = round_to_residue(HC, 16, p.W % 16);
    int cfg = -1;
    for (int nb = 1; nb <= 16 && cfg < 0; ++nb)
        if (HW <= 16 * nb) cfg = gi::img16_config(nb, p.kH, p.kW, HP, HR);
    if (cfg < 0) return false;
    // Slots past the image read position j16 + the tap shift: inside the plane.
    if (15 + (p.kH - 1) * HP + p.kW - 1 >= HR * HP) return false;
    const int nchunks = (p.Co + 31) / 32;
    const int wtiles = (p.Ci + 63) / 64;
    const int ci_tiles = (p.Ci + 127) / 128;
    const int64_t lim = 0x7fff0000LL;
    const int64_t wk = (int64_t)wtiles * nchunks * p.kH * p.kW * 4096;
    if (wk > lim || (int64_t)p.N * p.Co * oHW * 2 > lim ||
        (int64_t)p.N * p.Ci * HW * 4 > lim || (int64_t)p.N * ci_tiles > INT32_MAX)
        return false;
    const int PS = gi::img16_plane(cfg);
    const size_t lds = gi::img16_lds(cfg);
    if (lds > kLdsBytes) return false;
    gi::Img16Args &a = out.args;
    a = gi::Img16Args{};
    a.g_bytes = (uint32_t)((int64_t)p.N * p.Co * oHW * 2);
    a.wk_bytes = (uint32_t)wk;
    a.d_bytes = (uint32_t)((int64_t)p.N * p.Ci * HW * 4);
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.oH = p.oH;
    a.oW = p.oW;
    a.kH = p.kH;
    a.kW = p.kW;
    a.oy = p.kH - 1 - p.pad_h;
    a.ox = p.kW - 1 - p.pad_w;
    a.HR = HR;
    a.HC = HC;
    a.HP = HP;
    a.PS = PS;
    a.nchunks = nchunks;
    a.ci_tiles = ci_tiles;
    a.nq = oHW / 4;
    a.rcp_w = gi::recip16(p.W);
    a.rcp_ow = gi::recip16(p.oW);
    out.cfg = cfg;
    out.lds = lds;
    out.wk_bytes = (size_t)wk;
    out.wtiles = wtiles;
    return true;
}

// Column plan (fp32): Ci*kH*kW columns in at most kCol2imMaxBlocks blocks
// of 16, kCol2imMinCo < Co <= kCol2imMaxCo, kW <= 4*stride.  Chooses the
// TH x TW input tile that minimises ceil(work-groups / CUs) x the busiest
// wave's blocks of 16 grad_out positions (each a 16 x NBN MFMA product and
// its fold), the work-groups running one per compute unit.
bool plan_col2im(const conv2d_gi_params &p, Col2imPlan &out) {
    const int ncols = p.Ci * p.kH * p.kW;
    const int nbn = (ncols + 15) / 16;
    if (nbn > gi::kCol2imMaxBlocks || p.Co <= gi::kCol2imMinCo || p.Co > gi::kCol2imMaxCo ||
        p.stride > gi::kCol2imMaxStride || p.kW > 4 * p.stride)
        return false;
    const int64_t lim = 0x7fff0000LL;
    if ((int64_t)p.N * p.Co * p.oH * p.oW * 4 > lim) return false;
    if ((int64_t)p.N * p.Ci * p.H * p.W * 4 > lim) return false;
    if ((int64_t)p.Co * ncols * 4 > lim) return false;
    const int s = p.stride;
    const int r0 = p.kH - 1, c0 = (p.kW - 1 + 3) / 4 * 4;
    bool found = false;
    double best = 0;
    const int Wq = (p.W + 3) / 4 * 4;
    for (int TH = 1; TH <= p.H; ++TH) {
        // Only the smallest TH for each row-tile count.
        const int tiles_r = (p.H + TH - 1) / TH;
        if (TH > 1 && (p.H + TH - 2) / (TH - 1) == tiles_r) continue;
        for (int TW = 4; TW <= Wq; TW += 4) {
            const int tiles_c = (p.W + TW - 1) / TW;
            if (TW > 4 && (p.W + TW - 5) / (TW - 4) == tiles_c) continue;
            const int nq = (TH + p.kH - 2) / s + 1;   // grad_out rows meeting a tile
            const int ncq = (TW + p.kW - 2) / s + 1;  // and columns
            // Rows per wave: even, each half at least D = ceil(kH / stride).
            const int RW = std::max((nq + 3) / 4 + ((nq + 3) / 4 & 1), 2 * ((p.kH + s - 1) / s));
            if (ncq > 16 * gi::kCol2imBlocksPerRow) continue;
            const int ncb = gi::kCol2imBlocksPerRow;
            gi::Col2imArgs t{};
            t.Ci = p.Ci;
            t.ncols = ncols;
            t.stride = s;
            t.ws = gi::col2im_f32_stage_stride(ncols, s);
            t.LR = r0 + TH + p.kH - 1;
            gi::col2im_f32_layout(p.kH, p.kW, t.LR,
                                  std::max(c0 + TW + p.kW - 1,
                                           c0 + 16 * s * gi::kCol2imBlocksPerRow + p.kW),
                                  t.LP, t.plane);
            if (gi::col2im_f32_lds_bytes(t) > kLdsBytes) continue;
            const int64_t wgs = (int64_t)p.N * tiles_r * tiles_c;
            if (wgs > INT32_MAX) continue;
            const double per_wg =
                (double)RW * ncb * (16.0 * nbn * 32 + 400.0) + 6000.0;
            const double cost = (double)((wgs + kCUs - 1) / kCUs) * per_wg +
                                0.02 * (double)wgs * per_wg / kCUs;
            if (!found || cost < best) {
                found = true;
                best = cost;
                gi::Col2imArgs &a = out.args;
                a = gi::Col2imArgs{};
                a.TH = TH;
                a.TW = TW;
                a.tiles_r = tiles_r;
                a.tiles_c = tiles_c;
                a.RW = RW;
                a.LR = t.LR;
                a.LP = t.LP;
                a.plane = t.plane;
            }
        }
    }
    if (!found) return false;
    gi::Col2imArgs &a = out.args;
    a.g_bytes = (uint32_t)((int64_t)p.N * p.Co * p.oH * p.oW * 4);
    a.w_bytes = (uint32_t)((int64_t)p.Co * ncols * 4);
    a.d_bytes = (uint32_t)((int64_t)p.N * p.Ci * p.H * p.W * 4);
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.oH = p.oH;
    a.oW = p.oW;
    a.kH = p.kH;
    a.kW = p.kW;
    a.stride = p.stride;
    a.pad_h = p.pad_h;
    a.pad_w = p.pad_w;
    a.ncols = ncols;
    a.r0 = r0;
    a.c0 = c0;
    a.ws = gi::col2im_f32_stage_stride(ncols, p.stride);
    a.magic_khw = gi::recip16(p.kH * p.kW);
    a.magic_kw = gi::recip16(p.kW);
    a.wofs = gi::col2im_f32_weight_offset(a);
    out.lds = gi::col2im_f32_lds_bytes(a);
    return true;
}

// Small-Ci plan (fp32, Ci <= 4): 16 x 16 phase-grid tiles; phase groups of
// near-equal tap totals, run in sets of up to two per work-group over one
// grad_out halo.  Every phase's tap count must be one the kernel is built
// for, and every set's halo and taps must fit the kernel's staging.
bool plan_stem(const conv2d_gi_params &p, const std::vector<Phase> &phases, StemPlan &out) {
    if (p.Ci > 4 || phases.empty() || (int)phases.size() > gi::kMaxPhasesPerLaunch) return false;
    const int64_t lim = 0x7fff0000LL;
    if ((int64_t)p.N * p.Co * p.oH * p.oW * 4 > lim) return false;
    if ((int64_t)p.N * p.Ci * p.H * p.W * 4 > lim) return false;
    // Weight offsets: an out-of-range marker (the weight's size) plus a chunk
    // offset must stay below 2^32.
    if ((int64_t)p.Co * p.Ci * p.kH * p.kW * 4 > lim / 2) return false;
    gi::StemArgs &a = out.args;
    a = gi::StemArgs{};
    const int nchunks = (p.Co + 3) / 4;
    int maxHa = 0, maxWb = 0;
    for (size_t i = 0; i < phases.size(); ++i) {
        const Phase &ph = phases[i];
        if (!gi::stem_f32_taps_ok(ph.J_h * ph.J_w)) return false;
        maxHa = std::max(maxHa, ph.Ha);
        maxWb = std::max(maxWb, ph.Wb);
        gi::StemPhase &s = a.ph[i];
        s.rho_h = ph.rho_h;
        s.rho_w = ph.rho_w;
        s.q_h = ph.q_h;
        s.q_w = ph.q_w;
        s.r_h = ph.r_h;
        s.r_w = ph.r_w;
        s.J_h = ph.J_h;
        s.J_w = ph.J_w;
        s.Ha = ph.Ha;
        s.Wb = ph.Wb;
    }
    // Phase groups: the phases sorted by tap count, the largest paired with
    // the smallest, so the groups' tap totals are close.
    std::vector<int> order(phases.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(), [&](int x, int y) {
        return phases[x].J_h * phases[x].J_w > phases[y].J_h * phases[y].J_w;
    });
    const int np = (int)order.size();
    a.ngroups = 0;
    for (int lo = 0, hi = np - 1; lo <= hi; ++lo, --hi) {
        a.group[a.ngroups][0] = (int8_t)order[lo];
        a.group[a.ngroups][1] = (int8_t)(lo < hi ? order[hi] : -1);
        ++a.ngroups;
    }
    const int G = gi::kStemGroupsPerWg;
    a.nsets = (a.ngroups + G - 1) / G;
    const int waves = gi::stem_f32_waves(a.ngroups);
    // Per set: the halo covering every phase with taps (origin relative to
    // the tile: q - (J - 1) rows and columns; extent 16 + J - 1), each
    // phase's origin inside it, and the phase's first staged tap.
    int pitch = 1, rows = 0;
    for (int st = 0; st < a.nsets; ++st) {
        int oh = INT32_MAX, ow = INT32_MAX, eh = INT32_MIN, ew = INT32_MIN, taps = 0;
        for (int g = st * G; g < std::min(a.ngroups, (st + 1) * G); ++g)
            for (int k = 0; k < 2; ++k) {
                const int pi = a.group[g][k];
                if (pi < 0) continue;
                gi::StemPhase &s = a.ph[pi];
                s.tb = taps;
                taps += s.J_h * s.J_w;
                if (s.J_h * s.J_w == 0) continue;
                oh = std::min(oh, s.q_h - (s.J_h - 1));
                ow = std::min(ow, s.q_w - (s.J_w - 1));
                eh = std::max(eh, s.q_h + 16);
                ew = std::max(ew, s.q_w + 16);
            }
        if (taps > waves * gi::kStemTapsPerWave) return false;
        if (oh == INT32_MAX) {  // no phase of the set has taps: nothing to load
            a.set_org[st][0] = a.set_org[st][1] = 0;
            a.set_ext[st][0] = a.set_ext[st][1] = 0;
            continue;
        }
        a.set_org[st][0] = oh;
        a.set_org[st][1] = ow;
        a.set_ext[st][0] = eh - oh;
        a.set_ext[st][1] = ew - ow;
        pitch = std::max(pitch, ew - ow);
        rows = std::max(rows, eh - oh);
        for (int g = st * G; g < std::min(a.ngroups, (st + 1) * G); ++g)
            for (int k = 0; k < 2; ++k) {
                const int pi = a.group[g][k];
                if (pi < 0) continue;
                gi::StemPhase &s = a.ph[pi];
                s.dr = s.J_h * s.J_w ? s.q_h - (s.J_h - 1) - oh : 0;
                s.dc = s.J_h * s.J_w ? s.q_w - (s.J_w - 1) - ow : 0;
            }
    }
    // The fixed pitch when every halo fits it: its instance has compile-time
    // tap shifts.
    if (pitch <= gi::stem_f32_fixed_pitch() &&
        rows * gi::stem_f32_fixed_pitch() <=
            gi::stem_f32_halo_positions(gi::stem_f32_fixed_pitch()))
        pitch = gi::stem_f32_fixed_pitch();
    const int hpmax = gi::stem_f32_halo_positions(pitch);
    if (rows * pitch > hpmax) return false;
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.oH = p.oH;
    a.oW = p.oW;
    a.stride = p.stride;
    a.nphases = (int)phases.size();
    a.nchunks = nchunks;
    a.tiles_r = (maxHa + 15) / 16;
    a.tiles_c = (maxWb + 15) / 16;
    a.HPmax = hpmax;
    a.pitch = pitch;
    a.g_bytes = (uint32_t)((int64_t)p.N * p.Co * p.oH * p.oW * 4);
    a.d_bytes = (uint32_t)((int64_t)p.N * p.Ci * p.H * p.W * 4);
    a.kH = p.kH;
    a.kW = p.kW;
    a.w_bytes = (uint32_t)((int64_t)p.Co * p.Ci * p.kH * p.kW * 4);
    const int64_t units = (int64_t)p.N * a.tiles_r * a.tiles_c * a.nsets;
    if (4 * units > INT32_MAX) return false;
    // Units past the last whole wave of kCUs run as quarter tiles, so the
    // compute units' shares differ by at most a quarter tile, provided every
    // work-group still finds a slot in the first wave (4 per compute unit).
    const int64_t rem = units % kCUs;
    const int64_t nfull = units - rem;
    a.nfull = (int32_t)units;
    if (a.nsets == 1 && rem > 0 && nfull + 4 * rem <= 4LL * kCUs) a.nfull = (int32_t)nfull;
    out.ws_bytes = 0;  // the kernel reads the weight as given
    return true;
}

// Generic plan: phase-split gathered GEMM, launches of at most
// kMaxPhasesPerLaunch phases.
void plan_generic(const conv2d_gi_params &p, const std::vector<Phase> &phases, Plan &plan) {
    plan.variant = CONV2D_GI_VARIANT_GENERIC;
    plan.ws_bytes = (size_t)p.Co * p.Ci * p.kH * p.kW * (plan.bf16 ? 2 : 4);
    GemmArgs base{};
    base.N = p.N;
    base.Ci = p.Ci;
    base.H = p.H;
    base.W = p.W;
    base.Co = p.Co;
    base.kH = p.kH;
    base.kW = p.kW;
    base.stride = p.stride;
    base.oH = p.oH;
    base.oW = p.oW;
    base.ci_tiles = (p.Ci + gi::kGenericBM - 1) / gi::kGenericBM;
    for (size_t i = 0; i < phases.size(); i += gi::kMaxPhasesPerLaunch) {
        Launch L{};
        L.args = base;
        int tiles = 0;
        int np = 0;
        for (size_t k = i; k < phases.size() && np < gi::kMaxPhasesPerLaunch; ++k, ++np) {
            Phase ph = phases[k];
            ph.tile_begin = tiles;
            const int64_t npix = (int64_t)p.N * ph.Ha * ph.Wb;
            tiles += (int)((npix + gi::kGenericBN - 1) / gi::kGenericBN);
            L.args.ph[np] = ph;
        }
        L.args.nphases = np;
        L.tiles_x = tiles;
        plan.launches.push_back(L);
    }
}

Plan make_plan(const conv2d_gi_params &p, bool bf16) {
    Plan plan;
    plan.bf16 = bf16;
    std::vector<Phase> phases = make_phases(p);
    const int forced = g_variant;
    bool want_halo = !bf16 && p.Ci >= 16 &&
                     (forced == CONV2D_GI_VARIANT_HALO || forced == CONV2D_GI_VARIANT_AUTO);
    if (want_halo && plan_halo(p, phases, plan.halo)) {
        plan.variant = CONV2D_GI_VARIANT_HALO;
        plan.ws_bytes = (size_t)plan.halo.ws_floats * sizeof(float);
        return plan;
    }
    if (!bf16 && (forced == CONV2D_GI_VARIANT_COL2IM || forced == CONV2D_GI_VARIANT_AUTO) &&
        plan_col2im(p, plan.c2i)) {
        plan.variant = CONV2D_GI_VARIANT_COL2IM;
        return plan;
    }
    if (!bf16 && (forced == CONV2D_GI_VARIANT_STEM || forced == CONV2D_GI_VARIANT_AUTO) &&
        plan_stem(p, phases, plan.stem)) {
        plan.variant = CONV2D_GI_VARIANT_STEM;
        plan.ws_bytes = plan.stem.ws_bytes;
        return plan;
    }
    // 16-bit inputs: the whole-image kernel where it applies and fills the
    // chip (a work-group per image and 128 channels), or when the tile hook
    // asks for its 13 blocks; else the halo-tile kernel.
    if (bf16 && (forced == CONV2D_GI_VARIANT_HALO || forced == CONV2D_GI_VARIANT_AUTO) &&
        (g_tile_nb == 0 || g_tile_nb == 13) && plan_img16(p, plan.im) &&
        (g_tile_nb == 13 || (int64_t)p.N * plan.im.args.ci_tiles >= kCUs)) {
        plan.variant = CONV2D_GI_VARIANT_HALO;
        plan.img16 = true;
        plan.ws_bytes = plan.im.wk_bytes;
        return plan;
    }
    if (bf16 && (forced == CONV2D_GI_VARIANT_HALO || forced == CONV2D_GI_VARIANT_AUTO) &&
        g_tile_nb != 13 && plan_halo_bf16(p, plan.hb)) {
        plan.variant = CONV2D_GI_VARIANT_HALO;
        plan.ws_bytes = plan.hb.gp_bytes + plan.hb.wk_bytes;
        return plan;
    }
    plan_generic(p, phases, plan);
    return plan;
}

// dt: 0 fp32 inputs, 1 bf16, 2 fp16 (the 16-bit kinds share plans, prologues
// and kernels up to the MFMA instruction).
// ext_ws, when not null, is caller-provided scratch of ext_cap bytes used in
// place of the per-stream cache (no allocation, no cache lock); a plan that
// needs more returns CONV2D_GI_EUNSUPPORTED before any HIP call.
template <typename T>
int run(const T *grad_out, const T *weight, float *dst, const conv2d_gi_params *p,
        hipStream_t stream, int dt, void *ext_ws = nullptr, size_t ext_cap = 0) {
    const bool bf16 = dt != 0;   // a 16-bit input kind
    const bool f16 = dt == 2;
    int rc = validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!dst || !grad_out || !weight) return CONV2D_GI_EINVAL;

    Plan plan = make_plan(*p, bf16);
    if (ext_ws && plan.ws_bytes > ext_cap) return CONV2D_GI_EUNSUPPORTED;
    void *ws = nullptr;
    hipError_t e;
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e);
    std::unique_lock<std::recursive_mutex> lock(g_ws_mu, std::defer_lock);
    if (!ext_ws) lock.lock();
    if (plan.ws_bytes > 0) {
        if (ext_ws)
            ws = ext_ws;
        else
            e = workspace_for(dev, stream, plan.ws_bytes, &ws);
        if (e != hipSuccess) return fail_hip(e);
        const int kHW = p->kH * p->kW;
        if (plan.variant == CONV2D_GI_VARIANT_HALO && plan.img16) {
            e = gi::launch_weight_frag16((const uint16_t *)weight, (uint16_t *)ws, p->Co, p->Ci,
                                         kHW, plan.im.args.nchunks, plan.im.wtiles, stream);
        } else if (plan.variant == CONV2D_GI_VARIANT_HALO && bf16) {
            HaloBf16Plan &h = plan.hb;
            uint16_t *gp = (uint16_t *)ws;
            uint16_t *wk = (uint16_t *)((char *)ws + h.gp_bytes);
            e = gi::launch_prologues_bf16((const uint16_t *)grad_out, gp,
                                          (const uint16_t *)weight, wk, h.args, p->oH, p->oW,
                                          p->pad_h, p->pad_w, h.ci_tiles, stream);
        } else if (plan.variant == CONV2D_GI_VARIANT_HALO)
            e = gi::launch_weight_image_f32((const float *)weight, (float *)ws, plan.halo.args,
                                            p->kH, p->kW, plan.halo.ci_tiles,
                                            plan.halo.ws_floats, stream);
        else if (bf16)
            e = gi::launch_weight_tap_ci_co_bf16((const uint16_t *)weight, (uint16_t *)ws, p->Co,
                                                 p->Ci, kHW, stream);
        else
            e = gi::launch_weight_tap_co_ci_f32((const float *)weight, (float *)ws, p->Co, p->Ci,
                                                kHW, stream);
        if (e != hipSuccess) return fail_hip(e);
    }
    e = hipSuccess;
    // Profiling events, when set, take the main kernel's own start and end
    // timestamps (first and last launch when there are several).
    gi::KernelEvents ev;
    if (g_prof_begin && g_prof_end) ev = {g_prof_begin, g_prof_end};
    if (plan.variant == CONV2D_GI_VARIANT_COL2IM) {
        gi::Col2imArgs &a = plan.c2i.args;
        a.grad_out = (const float *)grad_out;
        a.w = (const float *)weight;
        a.dst = dst;
        e = gi::launch_col2im_f32(a, stream, ev);
    } else if (plan.variant == CONV2D_GI_VARIANT_STEM) {
        if (e == hipSuccess) {
            gi::StemArgs &a = plan.stem.args;
            a.grad_out = (const float *)grad_out;
            a.w = (const float *)weight;
            a.dst = dst;
            e = gi::launch_stem_f32(a, stream, ev);
        }
    } else if (plan.variant == CONV2D_GI_VARIANT_HALO && plan.img16) {
        if (e == hipSuccess) {
            Img16Plan &m = plan.im;
            m.args.g = (const uint16_t *)grad_out;
            m.args.wk = (const uint16_t *)ws;
            m.args.dst = dst;
            e = gi::launch_img16(m.args, m.cfg, f16, m.lds, stream, ev);
        }
    } else if (plan.variant == CONV2D_GI_VARIANT_HALO && bf16) {
        if (e == hipSuccess) {
            HaloBf16Plan &h = plan.hb;
            h.args.gp = (const uint16_t *)ws;
            h.args.wk = (const uint16_t *)((char *)ws + h.gp_bytes);
            h.args.dst = dst;
            e = f16 ? gi::launch_halo_f16(h.args, h.cfg, h.tiles, h.ci_tiles, h.lds, stream, ev)
                    : gi::launch_halo_bf16(h.args, h.cfg, h.tiles, h.ci_tiles, h.lds, stream, ev);
        }
    } else if (plan.variant == CONV2D_GI_VARIANT_HALO) {
        if (e == hipSuccess) {
            HaloPlan &h = plan.halo;
            h.args.grad_out = (const float *)grad_out;
            h.args.wk = (const float *)ws;
            h.args.dst = dst;
            e = gi::launch_halo_f32(h.args, h.cfg, h.tiles, h.ci_tiles, h.lds, stream, ev);
        }
    } else {
        const size_t nl = plan.launches.size();
        for (size_t i = 0; i < nl; ++i) {
            if (e != hipSuccess) break;
            Launch &L = plan.launches[i];
            L.args.grad_out = grad_out;
            L.args.wt = ws;
            L.args.dst = dst;
            gi::KernelEvents li;
            li.start = i == 0 ? ev.start : nullptr;
            li.stop = i + 1 == nl ? ev.stop : nullptr;
            e = f16    ? gi::launch_generic_f16(L.args, L.tiles_x, stream, li)
                : bf16 ? gi::launch_generic_bf16(L.args, L.tiles_x, stream, li)
                       : gi::launch_generic_f32(L.args, L.tiles_x, stream, li);
        }
    }
    if (e != hipSuccess) return fail_hip(e);
    return CONV2D_GI_OK;
}

// grad_weight plan (fp32): 64 output channels x 16 input channels x a group
// of kernel rows (at most gw_f32_max_taps() taps) per work-group; output
// rows in groups of RPC rows (about 64 padded pixels per group); the groups
// split into slices so the grid holds about two work-groups per compute unit.
struct GwPlan {
    gi::GwArgs args{};
    size_t ws_bytes = 0;   // partial sums: slices x Co x Ci x kH x kW floats
    size_t lds = 0;
};

bool plan_gw(const conv2d_gi_params &p, GwPlan &out) {
    const int64_t lim = 0x7fff0000LL;
    if ((int64_t)p.N * p.Co * p.oH * p.oW * 4 > lim) return false;
    if ((int64_t)p.N * p.Ci * p.H * p.W * 4 > lim) return false;
    if (p.kW > gi::gw_f32_max_taps()) return false;
    gi::GwArgs &a = out.args;
    a = gi::GwArgs{};
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.oH = p.oH;
    a.oW = p.oW;
    a.stride = p.stride;
    a.pad_h = p.pad_h;
    a.pad_w = p.pad_w;
    a.kH = p.kH;
    a.kW = p.kW;
    a.x_bytes = (uint32_t)((int64_t)p.N * p.Ci * p.H * p.W * 4);
    a.g_bytes = (uint32_t)((int64_t)p.N * p.Co * p.oH * p.oW * 4);
    a.co_blocks = (p.Co + 63) / 64;
    a.ci_blocks = (p.Ci + 15) / 16;
    a.khg = std::max(1, std::min(p.kH, gi::gw_f32_max_taps() / p.kW));
    a.tap_groups = (p.kH + a.khg - 1) / a.khg;
    const int OWP = 4 * ((p.oW + 3) / 4);
    if (OWP > 64 * gi::gw_f32_max_blocks()) return false;
    // Rows per group: about 64 padded pixels, fewer while the two LDS stages
    // do not fit; one stage (no overlap of loads and arithmetic) for a single
    // row that still does not fit.
    a.XP = (OWP - 1) * p.stride + p.kW;
    a.XPM = (a.XP + 63) / 64 * 64;
    bool fits = false;
    for (int rpc = std::max(1, std::min(p.oH, 64 / OWP)); rpc >= 1 && !fits; --rpc) {
        a.RPC = rpc;
        a.GM = (a.RPC * OWP + 63) / 64;
        a.XR = (a.RPC - 1) * p.stride + a.khg;
        a.CIP = a.XR * a.XPM + 4;
        for (int st = 2; st >= (rpc == 1 ? 1 : 2) && !fits; --st) {
            a.stages = st;
            out.lds = gi::gw_f32_lds_bytes(a);
            fits = out.lds <= (size_t)kLdsBytes;
        }
    }
    if (!fits) return false;
    a.groups_img = (p.oH + a.RPC - 1) / a.RPC;
    const int64_t groups = (int64_t)p.N * a.groups_img;
    const int64_t tiles = (int64_t)a.co_blocks * a.ci_blocks * a.tap_groups;
    int64_t slices = std::max<int64_t>(1, std::min<int64_t>(groups, (2 * kCUs + tiles - 1) / tiles));
    // An empty batch still writes dw (zeros): one slice of no groups.
    a.groups_slice = (int)std::max<int64_t>(1, (groups + slices - 1) / slices);
    slices = std::max<int64_t>(1, (groups + a.groups_slice - 1) / a.groups_slice);
    a.slices = (int)slices;
    if (tiles * slices > INT32_MAX) return false;
    const int64_t total = (int64_t)p.Co * p.Ci * p.kH * p.kW;
    if (total * 4 > lim) return false;
    out.ws_bytes = (size_t)(slices * total * 4);
    return true;
}

// grad_weight with 16-byte direct loads (gi_gwd_f32).  Layout and column
// map from the shape; then the rows per group, LDS stages and slices that
// minimise a cost model: MFMA cycles of the busiest compute unit (including
// the padding pixels of a layout), a per-group synchronisation cost that
// other work-groups on the compute unit hide, and the slice reduction's
// traffic.
struct GwdPlan {
    gi::GwdArgs args{};
    int cfg = -1;
    int occ = 0;           // work-groups per compute unit that fit in LDS
    size_t ws_bytes = 0;
    size_t lds = 0;
};

uint32_t div_magic(int d) {
    return d <= 1 ? 0u : (uint32_t)((1ULL << 32) / (uint64_t)d + 1);
}

// (m, k) of q = (s * m) >> k = floor(s / d) for 0 <= s < 2^14: 2^k >= 2^14 d,
// m = ceil(2^k / d) < 2^15, so s * m < 2^29 (one 24-bit multiply) and the
// error s * (m d - 2^k) / 2^k stays below s d / 2^k <= 1 (exact).
uint32_t div24(int d) {
    if (d < 1) return 0u;
    int k = 14;
    while ((1LL << k) < 16384LL * d) ++k;
    const uint64_t m = ((1ULL << k) + (uint64_t)d - 1) / (uint64_t)d;
    return (uint32_t)k << 24 | (uint32_t)m;
}

int odd_quads(int64_t n) {   // smallest multiple of 4 >= n whose quarter is odd
    int64_t v = (n + 3) / 4 * 4;
    if ((v / 4) % 2 == 0) v += 4;
    return (int)v;
}

bool plan_gwd(const conv2d_gi_params &p, GwdPlan &out, bool bias = false) {
    const int64_t lim = 0x7fff0000LL;
    if ((int64_t)p.N * p.Co * p.oH * p.oW * 4 > lim) return false;
    // Planes within the kernel's 24-bit multiplies.
    if ((int64_t)p.oH * p.oW >= (1 << 24) || (int64_t)p.H * p.W >= (1 << 24)) return false;
    if ((int64_t)p.N * p.Ci * p.H * p.W * 4 > lim) return false;
    const int64_t total = (int64_t)p.Co * p.Ci * p.kH * p.kW;
    if (total * 4 > lim) return false;
    const int64_t HW = (int64_t)p.H * p.W;
    const bool flat = p.stride == 1 && p.oH == p.H && p.oW == p.W && p.W >= 4 &&
                      (p.kW == 3 || p.kW == 7) && (HW % 4 == 0 || (p.kH == 1 && p.pad_h == 0));
    const bool rowpad = p.W % 4 == 0 && p.oW % 4 == 0;
    if (!flat && !rowpad) return false;
    gi::GwdArgs a{};
    a.N = p.N;
    a.Ci = p.Ci;
    a.H = p.H;
    a.W = p.W;
    a.Co = p.Co;
    a.oH = p.oH;
    a.oW = p.oW;
    a.stride = p.stride;
    a.pad_h = p.pad_h;
    a.pad_w = p.pad_w;
    a.kH = p.kH;
    a.kW = p.kW;
    a.x_bytes = (uint32_t)((int64_t)p.N * p.Ci * HW * 4);
    a.g_bytes = (uint32_t)((int64_t)p.N * p.Co * p.oH * p.oW * 4);
    a.flat = flat ? 1 : 0;
    a.plane_zero = flat && HW % 4 == 0 ? 1 : 0;
    a.co_blocks = (p.Co + 63) / 64;
    int cfg;
    if (flat) {
        // 3 x 3 on rows of at least 18 pixels: the instance whose K blocks
        // inside a row skip the column masks.
        cfg = p.kW == 3 ? (p.W >= 18 ? 6 : 0) : 1;
        a.colmap = 0;
        a.khg = p.kW == 3 ? 3 : 1;
    } else if (p.kW == 3 && (p.stride == 1 || p.stride == 2) && p.Ci >= 16) {
        cfg = p.stride == 1 ? 2 : 3;
        a.colmap = 0;
        a.khg = 3;
    } else {
        cfg = p.stride == 2 ? 4 : 5;
        a.colmap = 1;
    }
    const int NB = gi::gwd_f32_blocks(cfg);
    const int kHW = p.kH * p.kW;
    if (a.colmap == 0) {
        a.tap_groups = (p.kH + a.khg - 1) / a.khg;
        a.col_tiles = (p.Ci + 15) / 16 * a.tap_groups;
        a.XC = 16;
    } else {
        a.khg = p.kH;
        a.tap_groups = 1;
        a.col_tiles = (int)((total / p.Co + 16 * NB - 1) / (16 * NB));
        a.XC = 1;
        for (int t = 0; t < a.col_tiles; ++t) {
            const int64_t c0 = (int64_t)t * 16 * NB;
            const int64_t c1 = std::min<int64_t>(c0 + 16 * NB, (int64_t)p.Ci * kHW) - 1;
            a.XC = std::max<int>(a.XC, (int)(c1 / kHW - c0 / kHW + 1));
        }
    }
    if (!flat) {
        a.OWP = (p.oW + 15) / 16 * 16;
        a.XO = (p.pad_w + 3) / 4 * 4;
        a.XW = (a.XO - p.pad_w + (a.OWP - 1) * p.stride + p.kW + 3) / 4 * 4;
    } else {
        a.OWP = 16;
        a.XO = 0;
        a.XW = 4;
    }
    const int64_t tiles = (int64_t)a.co_blocks * a.col_tiles;
    bool found = false;
    double best = 0;
    for (int R = 1; R <= std::min(p.oH, 64); ++R) {
        if (g_gw_rows > 0 && R != std::min(g_gw_rows, p.oH)) continue;
        int64_t nkb, LA, LX;
        if (flat) {
            nkb = ((int64_t)R * p.oW + 15) / 16;
            LA = odd_quads(16 * nkb + 3);
            LX = odd_quads(16 * nkb + (int64_t)(a.khg - 1) * p.W + p.kW + 2);
        } else {
            nkb = (int64_t)R * (a.OWP / 16);
            LA = odd_quads((int64_t)R * a.OWP);
            LX = odd_quads((int64_t)((R - 1) * p.stride + a.khg) * a.XW);
        }
        const int64_t nslots = 16 * LA + a.XC * (LX / 4);
        const int64_t stage_floats = (nslots + 63) / 64 * 256;
        for (int stages = 2; stages >= 1; --stages) {
            if (g_gw_stages > 0 && stages != g_gw_stages) continue;
            const size_t lds = (size_t)stages * stage_floats * 4;
            if (lds > kLdsBytes) continue;
            const int occ = (int)std::min<size_t>(gi::gwd_f32_max_wgs(cfg), kLdsBytes / lds);
            const int64_t groups_img = (p.oH + R - 1) / R;
            const int64_t groups = (int64_t)p.N * groups_img;
            int64_t slices = std::max<int64_t>(
                1, std::min<int64_t>(groups, (occ * kCUs + tiles - 1) / tiles));
            if (g_gw_slices > 0) slices = std::min<int64_t>(slices, g_gw_slices);
            const int64_t gs = std::max<int64_t>(1, (groups + slices - 1) / slices);
            slices = std::max<int64_t>(1, (groups + gs - 1) / gs);
            if (tiles * slices > INT32_MAX) continue;
            const int64_t wgs = tiles * slices;
            const int64_t per_cu = (wgs + kCUs - 1) / kCUs;
            // One wave per SIMD leaves LDS and load latency exposed
            // (measured: about 0.7 of the MFMA rate); a single stage waits
            // for each group's loads, which a second work-group hides.  Two
            // stages carry the next group's loads through the K blocks
            // (registers and issue slots): with a second work-group they
            // measured no faster than one stage (strided downsample: 198.9
            // against 187.4 us with one stage and twice the rows).
            const double mfma = (double)nkb * 4 * NB * 32;         // cycles per group
            const double eff = occ >= 2 ? 1.0 : 0.7;
            const double sync = stages == 2 ? 900.0 : (occ >= 2 ? 800.0 : 3000.0);
            const double t_main = (double)per_cu * gs * mfma / eff +
                                  (double)gs * sync * (double)((per_cu + occ - 1) / occ);
            const double t_red = (double)slices * total * 8 * 2.4e9 / 4.0e12;
            const double cost = t_main + t_red;
            if (!found || cost < best) {
                found = true;
                best = cost;
                a.R = R;
                a.groups_img = (int)groups_img;
                a.groups_slice = (int)gs;
                a.slices = (int)slices;
                a.LA = (int)LA;
                a.LX = (int)LX;
                a.XR = (R - 1) * p.stride + a.khg;
                a.nslots = (int)nslots;
                a.stage_floats = (int)stage_floats;
                a.stages = stages;
                out.lds = lds;
                out.occ = occ;
            }
        }
    }
    if (!found) return false;
    if (flat) a.XR = 0;
    a.m_w = div_magic(p.W);
    a.d24_la4 = div24(a.LA / 4);
    a.d24_owp4 = div24(a.OWP / 4);
    a.d24_lx4 = div24(a.LX / 4);
    a.d24_xw4 = div24(a.XW / 4);
    out.args = a;
    out.cfg = cfg;
    out.args.bias = bias ? 1 : 0;
    out.args.part_stride = (int)(total + (bias ? p.Co : 0));
    out.ws_bytes = (size_t)((int64_t)a.slices * out.args.part_stride * 4);
    return true;
}

std::string describe_gwd(const GwdPlan &g) {
    const gi::GwdArgs &a = g.args;
    return "variant=gwd dtype=f32 ws_bytes=" + std::to_string(g.ws_bytes) +
           " launches=2 [cfg=" + std::to_string(g.cfg) +
           (a.flat ? " layout=flat" : " layout=rowpad") +
           (a.colmap ? " map=flattened" : " map=tap") + " tiles=" +
           std::to_string(a.co_blocks) + "x" + std::to_string(a.col_tiles) +
           " slices=" + std::to_string(a.slices) + " rows_per_group=" + std::to_string(a.R) +
           " groups_per_slice=" + std::to_string(a.groups_slice) +
           " stages=" + std::to_string(a.stages) + " lds=" + std::to_string(g.lds) +
           " occ=" + std::to_string(g.occ) + "]";
}

std::string describe_gw(const GwPlan &g) {
    const gi::GwArgs &a = g.args;
    return "variant=gw dtype=f32 ws_bytes=" + std::to_string(g.ws_bytes) +
           " launches=2 [tiles=" + std::to_string(a.co_blocks) + "x" +
           std::to_string(a.ci_blocks) + "x" + std::to_string(a.tap_groups) +
           " khg=" + std::to_string(a.khg) + " slices=" + std::to_string(a.slices) +
           " rows_per_group=" + std::to_string(a.RPC) + " groups_per_slice=" +
           std::to_string(a.groups_slice) + " stages=" + std::to_string(a.stages) +
           " lds=" + std::to_string(g.lds) + "]";
}

// dt: 0 fp32, 1 bf16, 2 fp16 inputs.
std::string describe(const Plan &plan, int dt) {
    const bool bf16 = dt != 0;
    std::string s = "variant=";
    s += plan.variant == CONV2D_GI_VARIANT_HALO   ? "halo"
         : plan.variant == CONV2D_GI_VARIANT_STEM ? "stem"
         : plan.variant == CONV2D_GI_VARIANT_COL2IM ? "col2im"
                                                  : "generic";
    s += " dtype=";
    s += dt == 2 ? "f16" : bf16 ? "bf16" : "f32";
    s += " ws_bytes=" + std::to_string(plan.ws_bytes);
    if (plan.variant == CONV2D_GI_VARIANT_COL2IM) {
        const gi::Col2imArgs &a = plan.c2i.args;
        s += " launches=1 [tile=" + std::to_string(a.TH) + "x" + std::to_string(a.TW) +
             " wgs=" + std::to_string((int64_t)a.N * a.tiles_r * a.tiles_c) +
             " cols=" + std::to_string(a.ncols) + " rows_per_wave=" + std::to_string(a.RW) +
             " lds=" + std::to_string(plan.c2i.lds) + " pitch=" + std::to_string(a.LP) +
             " plane=" + std::to_string(a.plane) + " stage=" + std::to_string(a.ws) + "]";
        return s;
    }
    if (plan.variant == CONV2D_GI_VARIANT_STEM) {
        const gi::StemArgs &a = plan.stem.args;
        s += " launches=1 [tiles=" + std::to_string(a.N) + "x" + std::to_string(a.tiles_r) + "x" +
             std::to_string(a.tiles_c) + "x" + std::to_string(a.nsets) +
             " whole=" + std::to_string(a.nfull) +
             " waves=" + std::to_string(gi::stem_f32_waves(a.ngroups)) +
             " pitch=" + std::to_string(a.pitch) + " chunks=" + std::to_string(a.nchunks);
        for (int i = 0; i < a.nphases; ++i) {
            const gi::StemPhase &ph = a.ph[i];
            s += " phase(" + std::to_string(ph.rho_h) + "," + std::to_string(ph.rho_w) +
                 ") taps=" + std::to_string(ph.J_h) + "x" + std::to_string(ph.J_w) +
                 " px=" + std::to_string(ph.Ha) + "x" + std::to_string(ph.Wb);
        }
        s += "]";
        return s;
    }
    if (plan.variant == CONV2D_GI_VARIANT_HALO && plan.img16) {
        const Img16Plan &m = plan.im;
        const gi::Img16Args &a = m.args;
        s += " launches=2 [image kernel cfg=" + std::to_string(m.cfg) +
             " nb=" + std::to_string(gi::img16_blocks(m.cfg)) + " wgs=" + std::to_string(a.N) +
             "x" + std::to_string(a.ci_tiles) + " lds=" + std::to_string(m.lds) +
             " halo=" + std::to_string(a.HR) + "x" + std::to_string(a.HC) + " pitch=" +
             std::to_string(a.HP) + " chunks=" + std::to_string(a.nchunks) + "]";
        return s;
    }
    if (plan.variant == CONV2D_GI_VARIANT_HALO && bf16) {
        const HaloBf16Plan &h = plan.hb;
        const gi::HaloBf16Args &a = h.args;
        s += " launches=2 [cfg=" + std::to_string(h.cfg) + " tile=" + std::to_string(a.TR) + "x" +
             std::to_string(a.TC) + " wgs=" + std::to_string(h.tiles) + "x" +
             std::to_string(h.ci_tiles) + " lds=" + std::to_string(h.lds) +
             " halo=" + std::to_string(a.HR) + "x" + std::to_string(a.HC) + " pitch=" +
             std::to_string(a.HP) +
             " chunks=" + std::to_string(a.nchunks) + "]";
        return s;
    }
    if (plan.variant == CONV2D_GI_VARIANT_HALO) {
        const HaloPlan &h = plan.halo;
        const gi::HaloArgs &a = h.args;
        s += " launches=1 [nb=" + std::to_string(h.nb) + " cfg=" + std::to_string(h.cfg) +
             (h.fused                     ? std::string(" fused")
              : gi::halo_f32_ks(h.cfg) > 1 ? " split=" + std::to_string(gi::halo_f32_ks(h.cfg))
                                           : std::string()) +
             " bl=" + std::to_string(h.bl) + " tile=" + std::to_string(a.TR) + "x" +
             std::to_string(a.TC) + (a.fold ? " fold" : "") + " wgs=" + std::to_string(h.tiles) +
             "x" + std::to_string(h.ci_tiles) + " lds=" + std::to_string(h.lds) +
             " HP=" + std::to_string(a.HP) + " HPc=" + std::to_string(a.HPc) +
             " stages=" + std::to_string(a.stages);
        for (int i = 0; i < a.nphases; ++i) {
            const gi::HaloPhase &ph = a.ph[i];
            s += " phase(" + std::to_string(ph.rho_h) + "," + std::to_string(ph.rho_w) +
                 ") taps=" + std::to_string(ph.J_h) + "x" + std::to_string(ph.J_w) +
                 " px=" + std::to_string(ph.Ha) + "x" + std::to_string(ph.Wb);
        }
        s += "]";
        return s;
    }
    s += " launches=" + std::to_string(plan.launches.size());
    for (const Launch &L : plan.launches) {
        s += " [tiles=" + std::to_string(L.tiles_x) + "x" + std::to_string(L.args.ci_tiles);
        for (int i = 0; i < L.args.nphases; ++i) {
            const Phase &ph = L.args.ph[i];
            s += " phase(" + std::to_string(ph.rho_h) + "," + std::to_string(ph.rho_w) +
                 ") taps=" + std::to_string(ph.J_h) + "x" + std::to_string(ph.J_w) +
                 " px=" + std::to_string(ph.Ha) + "x" + std::to_string(ph.Wb);
        }
        s += "]";
    }
    return s;
}

// Scratch floats of the bias gradient alone (per-channel partial sums).
size_t bias_ws_bytes(const conv2d_gi_params &p) {
    return (size_t)gi::channel_sum_blocks(p.N, p.Co, p.oH * p.oW) * p.Co * 4;
}

// grad_weight into dw and, when db is not null, the bias gradient into db:
// summed by the 16-byte-load kernel from the grad_out values it reads, else
// (the 4-byte-load kernel) by a separate per-channel pass.  Arguments are
// validated by the caller.
int run_gw_checked(const float *grad_out, const float *x, float *dw, float *db,
                   const conv2d_gi_params *p, hipStream_t stream) {
    const int variant = g_gw_variant;
    GwdPlan dplan;
    const bool use_d = variant != 1 && plan_gwd(*p, dplan, db != nullptr);
    if (variant == 2 && !use_d) return CONV2D_GI_EUNSUPPORTED;
    GwPlan plan;
    if (!use_d && !plan_gw(*p, plan)) return CONV2D_GI_EUNSUPPORTED;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e);
    std::lock_guard<std::recursive_mutex> lock(g_ws_mu);
    void *ws = nullptr;
    size_t need = use_d ? dplan.ws_bytes : plan.ws_bytes;
    if (!use_d && db) need = std::max(need, bias_ws_bytes(*p));
    e = workspace_for(dev, stream, need, &ws);
    if (e != hipSuccess) return fail_hip(e);
    gi::KernelEvents ev;
    if (g_prof_begin && g_prof_end) ev = {g_prof_begin, g_prof_end};
    if (use_d) {
        gi::GwdArgs &d = dplan.args;
        d.x = x;
        d.grad_out = grad_out;
        d.part = (float *)ws;
        d.dw = dw;
        d.db = db;
        e = gi::launch_gwd_f32(d, dplan.cfg, stream, ev);
        if (e != hipSuccess) return fail_hip(e);
        return CONV2D_GI_OK;
    }
    gi::GwArgs &a = plan.args;
    a.x = x;
    a.grad_out = grad_out;
    a.part = (float *)ws;
    a.dw = dw;
    e = gi::launch_gw_f32(a, stream, ev);
    if (e != hipSuccess) return fail_hip(e);
    if (db) {
        e = gi::launch_channel_sum(grad_out, (float *)ws, db, p->N, p->Co, p->oH * p->oW, stream);
        if (e != hipSuccess) return fail_hip(e);
    }
    return CONV2D_GI_OK;
}

int run_gw(const float *grad_out, const float *x, float *dw, const conv2d_gi_params *p,
           hipStream_t stream) {
    int rc = validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!dw || !grad_out || !x) return CONV2D_GI_EINVAL;
    return run_gw_checked(grad_out, x, dw, nullptr, p, stream);
}

// The bias gradient alone (arguments validated by the caller).
int run_bias_checked(const float *grad_out, float *db, const conv2d_gi_params *p,
                     hipStream_t stream) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e);
    std::lock_guard<std::recursive_mutex> lock(g_ws_mu);
    void *ws = nullptr;
    e = workspace_for(dev, stream, bias_ws_bytes(*p), &ws);
    if (e != hipSuccess) return fail_hip(e);
    e = gi::launch_channel_sum(grad_out, (float *)ws, db, p->N, p->Co, p->oH * p->oW, stream);
    if (e != hipSuccess) return fail_hip(e);
    return CONV2D_GI_OK;
}

int run_backward(const float *grad_out, const float *x, const float *weight, float *dx,
                 float *dw, float *db, const conv2d_gi_params *p, hipStream_t stream) {
    int rc = validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    // Every requested output needs grad_out; dx needs the weight, dw the input.
    if ((dx || dw || db) && !grad_out) return CONV2D_GI_EINVAL;
    if (dx && !weight) return CONV2D_GI_EINVAL;
    if (dw && !x) return CONV2D_GI_EINVAL;
    if (dx) {
        rc = run<float>(grad_out, weight, dx, p, stream, 0);
        if (rc != CONV2D_GI_OK) return rc;
    }
    if (dw) return run_gw_checked(grad_out, x, dw, db, p, stream);
    if (db) return run_bias_checked(grad_out, db, p, stream);
    return CONV2D_GI_OK;
}

// The forward convolution.  Stride 1 with pad <= k-1 runs on the grad_input
// path: y = sum over ci, kh, kw of x[oh-ph+kh, ow-pw+kw] * w[co,ci,kh,kw] is,
// with kh' = kH-1-kh, the grad_input sum of grad_out := x (Ci channels) and
// weight wf[ci][co][kh'][kw'] = w[co][ci][kH-1-kh'][kW-1-kw'] under the pad
// kH-1-ph (and kW-1-pw): an input-side problem with Ci' = Co, H' = oH,
// Co' = Ci, oH' = H.  Other shapes run on the generic forward kernel.
bool fwd_via_grad_input(const conv2d_gi_params &p) {
    return g_fwd_variant != 2 && p.stride == 1 && p.pad_h <= p.kH - 1 &&
           p.pad_w <= p.kW - 1;
}

conv2d_gi_params fwd_as_grad_input(const conv2d_gi_params &p) {
    conv2d_gi_params q{};
    q.N = p.N;
    q.Ci = p.Co;
    q.H = p.oH;
    q.W = p.oW;
    q.Co = p.Ci;
    q.kH = p.kH;
    q.kW = p.kW;
    q.stride = 1;
    q.pad_h = p.kH - 1 - p.pad_h;
    q.pad_w = p.kW - 1 - p.pad_w;
    q.oH = p.H;
    q.oW = p.W;
    return q;
}

int run_forward(const float *x, const float *w, float *y, const conv2d_gi_params *p,
                hipStream_t stream) {
    int rc = validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!y || !x || !w) return CONV2D_GI_EINVAL;
    const int64_t n_w = (int64_t)p->Co * p->Ci * p->kH * p->kW;
    if (g_fwd_variant == 1 && !fwd_via_grad_input(*p)) return CONV2D_GI_EUNSUPPORTED;
    const int kHW = p->kH * p->kW;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e);
    if (fwd_via_grad_input(*p)) {
        const conv2d_gi_params q = fwd_as_grad_input(*p);
        rc = validate(&q);
        if (rc != CONV2D_GI_OK) return rc;
        void *wf = nullptr;
        // Held across the grad_input call too: another thread enqueueing a
        // forward on this stream in between would overwrite slot 1.
        std::lock_guard<std::recursive_mutex> lock(g_ws_mu);
        e = workspace_for(dev, stream, (size_t)std::max<int64_t>(n_w, 1) * 4, &wf, 1);
        if (e != hipSuccess) return fail_hip(e);
        if (n_w > 0) {
            e = gi::launch_fwd_weight_flip_f32(w, (float *)wf, p->Co, p->Ci, kHW, stream);
            if (e != hipSuccess) return fail_hip(e);
        }
        return run<float>(x, (const float *)wf, y, &q, stream, 0);
    }
    std::lock_guard<std::recursive_mutex> lock(g_ws_mu);
    void *ws = nullptr;
    e = workspace_for(dev, stream, (size_t)(n_w + gi::kFwdZeroTail) * 4, &ws);
    if (e != hipSuccess) return fail_hip(e);
    gi::FwdArgs a{};
    a.x = x;
    a.wt = (const float *)ws;
    a.zero = (const float *)ws + n_w;
    a.y = y;
    a.N = p->N;
    a.Ci = p->Ci;
    a.H = p->H;
    a.W = p->W;
    a.Co = p->Co;
    a.kH = p->kH;
    a.kW = p->kW;
    a.stride = p->stride;
    a.pad_h = p->pad_h;
    a.pad_w = p->pad_w;
    a.oH = p->oH;
    a.oW = p->oW;
    if (n_w > 0) {
        e = gi::fwd_flat_k(a)
                ? gi::launch_fwd_weight_k_co_f32(w, (float *)ws, p->Co, p->Ci * kHW, stream)
                : gi::launch_fwd_weight_tap_ci_co_f32(w, (float *)ws, p->Co, p->Ci, kHW, stream);
        if (e != hipSuccess) return fail_hip(e);
    }
    gi::KernelEvents ev;
    if (g_prof_begin && g_prof_end) ev = {g_prof_begin, g_prof_end};
    e = gi::launch_fwd_generic_f32(a, stream, ev);
    if (e != hipSuccess) return fail_hip(e);
    return CONV2D_GI_OK;
}

std::string describe_forward(const conv2d_gi_params &p) {
    if (fwd_via_grad_input(p)) {
        const conv2d_gi_params q = fwd_as_grad_input(p);
        return describe(make_plan(q, false), false) + " (forward as grad_input: weight "
               "transposed and reversed)";
    }
    const int64_t npix = (int64_t)p.N * p.oH * p.oW;
    return "variant=fwd dtype=f32 ws_bytes=" +
           std::to_string(((int64_t)p.Co * p.Ci * p.kH * p.kW + gi::kFwdZeroTail) * 4) +
           " launches=2 [tiles=" +
           std::to_string((npix + gi::kFwdBN - 1) / gi::kFwdBN) + "x" +
           std::to_string((p.Co + gi::kFwdBM - 1) / gi::kFwdBM) + "]";
}

}  // namespace

namespace gi {

int record_hip_error(hipError_t e) { return fail_hip(e); }

// Scratch bytes the fp32 grad_input plan for p needs (0 when the shape is
// invalid); host only.
size_t grad_input_f32_scratch_bytes(const conv2d_gi_params &p) {
    if (validate(&p) != CONV2D_GI_OK) return 0;
    return make_plan(p, false).ws_bytes;
}

// fp32 grad_input on caller-provided device scratch (cap bytes): nothing is
// allocated and the per-stream cache is not touched.
int grad_input_f32_on_scratch(const float *grad_out, const float *weight, float *dst,
                              const conv2d_gi_params &p, hipStream_t stream, void *scratch,
                              size_t cap) {
    if (!scratch) return CONV2D_GI_EINVAL;
    return run<float>(grad_out, weight, dst, &p, stream, 0, scratch, cap);
}

}  // namespace gi

extern "C" {

int conv2d_forward(const float *x, const float *w, float *y, conv2d_gi_params p,
                   hipStream_t stream) {
    return run_forward(x, w, y, &p, stream);
}

int conv2d_fwd_plan(conv2d_gi_params p, char *buf, size_t len) {
    int rc = validate(&p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!buf || len == 0) return CONV2D_GI_EINVAL;
    if (g_fwd_variant == 1 && !fwd_via_grad_input(p)) return CONV2D_GI_EUNSUPPORTED;
    std::snprintf(buf, len, "%s", describe_forward(p).c_str());
    return CONV2D_GI_OK;
}

int conv2d_fwd_set_variant(int mode) {
    if (mode < 0 || mode > 2) return CONV2D_GI_EINVAL;
    g_fwd_variant = mode;
    return CONV2D_GI_OK;
}

int conv2d_grad_weight(const float *grad_out, const float *x, float *dw,
                       conv2d_gi_params p, hipStream_t stream) {
    return run_gw(grad_out, x, dw, &p, stream);
}

int conv2d_backward(const float *grad_out, const float *x, const float *weight, float *dx,
                    float *dw, float *db, conv2d_gi_params p, hipStream_t stream) {
    return run_backward(grad_out, x, weight, dx, dw, db, &p, stream);
}

int conv2d_grad_bias(const float *grad_out, float *db, conv2d_gi_params p,
                     hipStream_t stream) {
    int rc = validate(&p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!db) return CONV2D_GI_EINVAL;
    return run_backward(grad_out, nullptr, nullptr, nullptr, nullptr, db, &p, stream);
}

int conv2d_gw_plan(conv2d_gi_params p, char *buf, size_t len) {
    int rc = validate(&p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!buf || len == 0) return CONV2D_GI_EINVAL;
    const int variant = g_gw_variant;
    GwdPlan dplan;
    if (variant != 1 && plan_gwd(p, dplan)) {
        std::snprintf(buf, len, "%s", describe_gwd(dplan).c_str());
        return CONV2D_GI_OK;
    }
    if (variant == 2) return CONV2D_GI_EUNSUPPORTED;
    GwPlan plan;
    if (!plan_gw(p, plan)) return CONV2D_GI_EUNSUPPORTED;
    std::snprintf(buf, len, "%s", describe_gw(plan).c_str());
    return CONV2D_GI_OK;
}

int conv2d_gw_set_tile(int rows, int stages, int max_slices) {
    if (rows < 0 || stages < 0 || stages > 2 || max_slices < 0) return CONV2D_GI_EINVAL;
    g_gw_rows = rows;
    g_gw_stages = stages;
    g_gw_slices = max_slices;
    return CONV2D_GI_OK;
}

int conv2d_gw_set_variant(int mode) {
    if (mode < 0 || mode > 2) return CONV2D_GI_EINVAL;
    g_gw_variant = mode;
    return CONV2D_GI_OK;
}

int conv2d_grad_input(const float *grad_out, const float *weight, float *dst,
                      conv2d_gi_params p, hipStream_t stream) {
    return run<float>(grad_out, weight, dst, &p, stream, 0);
}

int conv2d_grad_input_bf16(const uint16_t *grad_out, const uint16_t *weight, float *dst,
                           conv2d_gi_params p, hipStream_t stream) {
    return run<uint16_t>(grad_out, weight, dst, &p, stream, 1);
}

int conv2d_grad_input_f16(const uint16_t *grad_out, const uint16_t *weight, float *dst,
                          conv2d_gi_params p, hipStream_t stream) {
    return run<uint16_t>(grad_out, weight, dst, &p, stream, 2);
}

int conv2d_gi_validate(conv2d_gi_params p) { return validate(&p); }

const char *conv2d_gi_strerror(int code) {
    switch (code) {
        case CONV2D_GI_OK: return "success";
        case CONV2D_GI_EINVAL: return "invalid argument (null pointer or inconsistent shape)";
        case CONV2D_GI_EUNSUPPORTED:
            return "shape the library does not serve (32-bit index width or kernel limits)";
        case CONV2D_GI_EHIP: return "HIP runtime error";
        default: return "unknown status code";
    }
}

const char *conv2d_gi_last_hip_error(void) { return g_last_hip; }

int conv2d_gi_set_variant(int variant) {
    if (variant != CONV2D_GI_VARIANT_AUTO && variant != CONV2D_GI_VARIANT_GENERIC &&
        variant != CONV2D_GI_VARIANT_HALO && variant != CONV2D_GI_VARIANT_STEM &&
        variant != CONV2D_GI_VARIANT_COL2IM)
        return -1;
    const int old = g_variant;
    g_variant = variant;
    return old;
}

int conv2d_gi_plan(conv2d_gi_params p, int dtype_bf16, char *buf, size_t len) {
    int rc = validate(&p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!buf || len == 0) return CONV2D_GI_EINVAL;
    if (dtype_bf16 < 0 || dtype_bf16 > 2) return CONV2D_GI_EINVAL;
    Plan plan = make_plan(p, dtype_bf16 != 0);
    std::snprintf(buf, len, "%s", describe(plan, dtype_bf16).c_str());
    return CONV2D_GI_OK;
}

int conv2d_gi_set_halo_tile(int nb, int tile_rows, int tile_cols, int stages) {
    if (nb == 0) {
        g_tile_nb = 0;
        g_tile_tr = 0;
        g_tile_tc = 0;
        g_tile_stages = 0;
        return CONV2D_GI_OK;
    }
    // fp32 takes nb in {4, 8, 13} (blocks per work-group), bf16 nb in {4, 7}
    // (blocks per wave, two waves across the tile).
    const int most_px = (nb == 4 || nb == 7) ? 2 * nb * 16 : nb * 16;
    if ((nb != 4 && nb != 7 && nb != 8 && nb != 13) || tile_rows < 1 || tile_cols < 1 ||
        tile_rows * tile_cols > most_px || stages < 0 || stages == 1 || stages > 3)
        return CONV2D_GI_EINVAL;
    g_tile_tr = tile_rows;
    g_tile_tc = tile_cols;
    g_tile_stages = stages;
    g_tile_nb = nb;
    return CONV2D_GI_OK;
}

int conv2d_gi_set_halo_fusion(int mode) {
    if (mode < 0 || mode > 2) return CONV2D_GI_EINVAL;
    g_halo_fusion = mode;
    return CONV2D_GI_OK;
}

int conv2d_gi_set_halo_split(int groups) {
    if (groups < 0 || groups > 2) return CONV2D_GI_EINVAL;
    g_halo_split = groups;
    return CONV2D_GI_OK;
}

int conv2d_gi_release_workspaces(void) {
    std::lock_guard<std::recursive_mutex> lock(g_ws_mu);
    int prev = 0;
    if (hipGetDevice(&prev) != hipSuccess) return fail_hip(hipErrorNoDevice);
    hipError_t first = hipSuccess;
    for (auto &kv : g_ws) {
        if (!kv.second.ptr) continue;
        hipError_t e = hipSetDevice(std::get<0>(kv.first));
        if (e == hipSuccess) e = hipFreeAsync(kv.second.ptr, std::get<1>(kv.first));
        if (e == hipSuccess) e = hipStreamSynchronize(std::get<1>(kv.first));
        if (first == hipSuccess) first = e;
    }
    g_ws.clear();
    (void)hipSetDevice(prev);
    return first == hipSuccess ? CONV2D_GI_OK : fail_hip(first);
}

void conv2d_gi_set_profile_events(hipEvent_t begin, hipEvent_t end) {
    g_prof_begin = begin;
    g_prof_end = end;
}

const char *conv2d_gi_version(void) { return "0.1.0"; }

}  // extern "C"
