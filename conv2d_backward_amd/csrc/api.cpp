// api.cpp -- the C ABI: argument checks, the planner and the launch sequence.
//
// Entry points and their contract are declared in include/conv2d_grad_input.h.
// Shape fields mirror the Params block of meganeura conv2d_grad_input_gemm.wgsl
// and the options of doppler conv2d_backward.d.ts (Conv2DBackwardOptions).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "conv2d_grad_input.h"
#include "gi_common.h"
#include "gi_launch.h"

namespace {

using gi::GemmArgs;
using gi::Phase;

std::atomic<int> g_variant{CONV2D_GI_VARIANT_AUTO};
thread_local char g_last_hip[256] = "";
thread_local hipEvent_t g_prof_begin = nullptr, g_prof_end = nullptr;

int fail_hip(hipError_t e) {
    std::snprintf(g_last_hip, sizeof(g_last_hip), "%s: %s", hipGetErrorName(e),
                  hipGetErrorString(e));
    return CONV2D_GI_EHIP;
}

int64_t floordiv(int64_t a, int64_t b) {  // b > 0
    return a >= 0 ? a / b : -((-a + b - 1) / b);
}

int validate(const conv2d_gi_params *p) {
    if (!p) return CONV2D_GI_EINVAL;
    if (p->N < 0 || p->Ci < 0 || p->Co < 0) return CONV2D_GI_EINVAL;
    if (p->H < 1 || p->W < 1 || p->kH < 1 || p->kW < 1 || p->stride < 1) return CONV2D_GI_EINVAL;
    if (p->pad_h < 0 || p->pad_w < 0) return CONV2D_GI_EINVAL;
    const int64_t oH = floordiv((int64_t)p->H + 2LL * p->pad_h - p->kH, p->stride) + 1;
    const int64_t oW = floordiv((int64_t)p->W + 2LL * p->pad_w - p->kW, p->stride) + 1;
    if (oH < 1 || oW < 1) return CONV2D_GI_EINVAL;
    if (p->oH != oH || p->oW != oW) return CONV2D_GI_EINVAL;
    // Index width: per-image planes, the weight and the folded pixel axis are
    // addressed with 32-bit offsets inside the kernels; batch offsets are 64-bit.
    const int64_t lim = INT32_MAX;
    if ((int64_t)p->Ci * p->H * p->W > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->Co * oH * oW > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->Co * p->Ci * p->kH * p->kW > lim) return CONV2D_GI_EUNSUPPORTED;
    if ((int64_t)p->N * p->H * p->W > lim) return CONV2D_GI_EUNSUPPORTED;
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

struct Plan {
    int variant = CONV2D_GI_VARIANT_GENERIC;
    bool bf16 = false;
    size_t ws_bytes = 0;  // reordered weight
    std::vector<Launch> launches;
};

Plan make_plan(const conv2d_gi_params &p, bool bf16) {
    Plan plan;
    plan.bf16 = bf16;
    plan.variant = CONV2D_GI_VARIANT_GENERIC;  // the only variant so far
    plan.ws_bytes = (size_t)p.Co * p.Ci * p.kH * p.kW * (bf16 ? 2 : 4);
    std::vector<Phase> phases = make_phases(p);
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
    return plan;
}

bool has_elems(int64_t n) { return n > 0; }

template <typename T>
int run(const T *grad_out, const T *weight, float *dst, const conv2d_gi_params *p,
        hipStream_t stream, bool bf16) {
    int rc = validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    const int64_t n_dst = (int64_t)p->N * p->Ci * p->H * p->W;
    const int64_t n_g = (int64_t)p->N * p->Co * p->oH * p->oW;
    const int64_t n_w = (int64_t)p->Co * p->Ci * p->kH * p->kW;
    if ((has_elems(n_dst) && !dst) || (has_elems(n_g) && !grad_out) ||
        (has_elems(n_w) && !weight))
        return CONV2D_GI_EINVAL;
    if (n_dst == 0) return CONV2D_GI_OK;

    Plan plan = make_plan(*p, bf16);
    void *ws = nullptr;
    hipError_t e;
    if (plan.ws_bytes > 0) {
        e = hipMallocAsync(&ws, plan.ws_bytes, stream);
        if (e != hipSuccess) return fail_hip(e);
        const int kHW = p->kH * p->kW;
        if (bf16)
            e = gi::launch_weight_tap_ci_co_bf16((const uint16_t *)weight, (uint16_t *)ws, p->Co,
                                                 p->Ci, kHW, stream);
        else
            e = gi::launch_weight_tap_co_ci_f32((const float *)weight, (float *)ws, p->Co, p->Ci,
                                                kHW, stream);
        if (e != hipSuccess) {
            (void)hipFreeAsync(ws, stream);
            return fail_hip(e);
        }
    }
    e = hipSuccess;
    if (g_prof_begin && g_prof_end) e = hipEventRecord(g_prof_begin, stream);
    for (Launch &L : plan.launches) {
        if (e != hipSuccess) break;
        L.args.grad_out = grad_out;
        L.args.wt = ws;
        L.args.dst = dst;
        e = bf16 ? gi::launch_generic_bf16(L.args, L.tiles_x, stream)
                 : gi::launch_generic_f32(L.args, L.tiles_x, stream);
    }
    if (e == hipSuccess && g_prof_begin && g_prof_end) e = hipEventRecord(g_prof_end, stream);
    if (ws) {
        hipError_t e2 = hipFreeAsync(ws, stream);
        if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return fail_hip(e);
    return CONV2D_GI_OK;
}

}  // namespace

extern "C" {

int conv2d_grad_input(const float *grad_out, const float *weight, float *dst,
                      const conv2d_gi_params *p, hipStream_t stream) {
    return run<float>(grad_out, weight, dst, p, stream, false);
}

int conv2d_grad_input_bf16(const uint16_t *grad_out, const uint16_t *weight, float *dst,
                           const conv2d_gi_params *p, hipStream_t stream) {
    return run<uint16_t>(grad_out, weight, dst, p, stream, true);
}

int conv2d_gi_validate(const conv2d_gi_params *p) { return validate(p); }

const char *conv2d_gi_strerror(int code) {
    switch (code) {
        case CONV2D_GI_OK: return "success";
        case CONV2D_GI_EINVAL: return "invalid argument (null pointer or inconsistent shape)";
        case CONV2D_GI_EUNSUPPORTED: return "shape beyond the library's 32-bit index width";
        case CONV2D_GI_EHIP: return "HIP runtime error";
        default: return "unknown status code";
    }
}

const char *conv2d_gi_last_hip_error(void) { return g_last_hip; }

int conv2d_gi_set_variant(int variant) {
    if (variant != CONV2D_GI_VARIANT_AUTO && variant != CONV2D_GI_VARIANT_GENERIC) return -1;
    return g_variant.exchange(variant);
}

int conv2d_gi_plan(const conv2d_gi_params *p, int dtype_bf16, char *buf, size_t len) {
    int rc = validate(p);
    if (rc != CONV2D_GI_OK) return rc;
    if (!buf || len == 0) return CONV2D_GI_EINVAL;
    Plan plan = make_plan(*p, dtype_bf16 != 0);
    std::string s = "variant=generic dtype=";
    s += dtype_bf16 ? "bf16" : "f32";
    s += " ws_bytes=" + std::to_string(plan.ws_bytes);
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
    std::snprintf(buf, len, "%s", s.c_str());
    return CONV2D_GI_OK;
}

void conv2d_gi_set_profile_events(hipEvent_t begin, hipEvent_t end) {
    g_prof_begin = begin;
    g_prof_end = end;
}

const char *conv2d_gi_version(void) { return "0.1.0"; }

}  // extern "C"
