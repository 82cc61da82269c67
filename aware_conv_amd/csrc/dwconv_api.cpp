// C-ABI front end of the plain depthwise conv baseline: argument checks
// (before anything is enqueued), then the whole-plane kernels with no
// wavelet levels and no base scale.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dwconv.h"
#include "wtconv_internal.h"

namespace {

using wtc::Grads;
using wtc::Params;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return n > 0 && x < y + n && y < x + n;
}

size_t elem_size(int dtype) { return dtype == WTCONV_F32 ? 4 : 2; }

// Checks the shape and fills the internal one (no levels).
int internal_shape(const dwconv_shape* d, wtconv_shape* s) {
    if (!d) return WTCONV_ERR_NULL;
    if (d->B < 0 || d->C < 0 || d->H < 0 || d->W < 0) return WTCONV_ERR_SHAPE;
    if (d->k < 1 || d->k > 7 || (d->k % 2) == 0) return WTCONV_ERR_KERNEL;
    if (d->dtype != WTCONV_F32 && d->dtype != WTCONV_F16) return WTCONV_ERR_DTYPE;
    if (d->H > (1 << 24) || d->W > (1 << 24)) return WTCONV_ERR_SHAPE;
    const unsigned long long n = (unsigned long long)d->B * (unsigned long long)d->C *
                                 (unsigned long long)d->H * (unsigned long long)d->W;
    if (d->H > 0 && d->W > 0 &&
        n / ((unsigned long long)d->H * d->W) != (unsigned long long)d->B * d->C)
        return WTCONV_ERR_SHAPE;
    if (n > (1ULL << 40)) return WTCONV_ERR_SHAPE;
    *s = wtconv_shape{d->B, d->C, d->H, d->W, 0, d->k, d->dtype};
    return WTCONV_OK;
}

bool empty_act(const wtconv_shape& s) { return s.B == 0 || s.C == 0 || s.H == 0 || s.W == 0; }

size_t act_bytes(const wtconv_shape& s) {
    return size_t(s.B) * s.C * s.H * s.W * elem_size(s.dtype);
}

int check_param(const void* p, int dtype) {
    if (!p) return WTCONV_ERR_NULL;
    return aligned(p, elem_size(dtype)) ? WTCONV_OK : WTCONV_ERR_ALIGN;
}

int hip_status(hipError_t e) { return e == hipSuccess ? WTCONV_OK : WTCONV_ERR_HIP; }

}  // namespace

extern "C" {

int dwconv_workspace_size(const dwconv_shape* d, size_t* bytes) {
    wtconv_shape s;
    int rc = internal_shape(d, &s);
    if (rc) return rc;
    if (!bytes) return WTCONV_ERR_NULL;
    if (empty_act(s)) {
        *bytes = 0;
        return WTCONV_OK;
    }
    if (!wtc::plane_supported(s)) return WTCONV_ERR_UNSUPPORTED;
    *bytes = wtc::plane_workspace_bytes(s);
    return WTCONV_OK;
}

int dwconv_fwd(const dwconv_shape* d, const void* x, const void* w, const void* bias, void* y,
               void* stream) {
    wtconv_shape s;
    int rc = internal_shape(d, &s);
    if (rc) return rc;
    if (s.C == 0) return WTCONV_OK;
    if ((rc = check_param(w, s.dtype)) || (rc = check_param(bias, s.dtype))) return rc;
    if (empty_act(s)) return WTCONV_OK;
    if (!x || !y) return WTCONV_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16)) return WTCONV_ERR_ALIGN;
    if (overlap(x, y, act_bytes(s))) return WTCONV_ERR_ALIAS;
    if (!wtc::plane_supported(s)) return WTCONV_ERR_UNSUPPORTED;
    Params p{w, bias, nullptr, nullptr, nullptr};
    return hip_status(wtc::plane_apply(s, x, p, y, false, static_cast<hipStream_t>(stream),
                                       wtc::Rag{s.H, s.W}));
}

int dwconv_bwd(const dwconv_shape* d, const void* x, const void* dy, const void* w, void* dx,
               void* dw, void* db, void* workspace, size_t ws_bytes, void* stream) {
    wtconv_shape s;
    int rc = internal_shape(d, &s);
    if (rc) return rc;
    if (s.C == 0) return WTCONV_OK;
    if ((rc = check_param(w, s.dtype)) || (rc = check_param(dw, s.dtype)) ||
        (rc = check_param(db, s.dtype)))
        return rc;
    // the bias is not needed for any gradient: w stands in for it
    Params p{w, w, nullptr, nullptr, nullptr};
    Grads g{dw, db, nullptr, nullptr, nullptr};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (empty_act(s)) return hip_status(wtc::zero_grads(s, p, g, st));
    if (!x || !dy || !dx) return WTCONV_ERR_NULL;
    if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16)) return WTCONV_ERR_ALIGN;
    if (overlap(dx, dy, act_bytes(s)) || overlap(dx, x, act_bytes(s))) return WTCONV_ERR_ALIAS;
    if (!wtc::plane_supported(s)) return WTCONV_ERR_UNSUPPORTED;
    const size_t need = wtc::plane_workspace_bytes(s);
    if (ws_bytes < need) return WTCONV_ERR_WORKSPACE;
    if (need > 0 && !workspace) return WTCONV_ERR_NULL;
    if (need > 0 && !aligned(workspace, 16)) return WTCONV_ERR_ALIGN;
    return hip_status(wtc::plane_bwd(s, x, dy, p, dx, g, workspace, st, wtc::Rag{s.H, s.W}));
}

}  // extern "C"
