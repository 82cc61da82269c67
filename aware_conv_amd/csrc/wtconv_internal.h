// Internal interface between the C-ABI front end (wtconv_api.cpp) and the
// kernel translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "wtconv.h"

namespace wtc {

// Raw (unfolded) parameter pointers, all in the layer's storage dtype.
struct Params {
    const void* w_base;  // [C][k][k]
    const void* b_base;  // [C]   (may be NULL for the input gradient)
    const void* s_base;  // [C]
    const void* w_wav;   // [L][C][4][k][k]
    const void* s_wav;   // [L][C][4]
};

struct Grads {
    void* dw_base;
    void* db_base;
    void* ds_base;
    void* dw_wav;
    void* ds_wav;
};

// The planes as stored in device memory, when they are smaller than the
// planes a whole-plane kernel computes on (Hs <= H, Ws <= W): the kernel
// reads them as the top-left corner of its planes, zero elsewhere (each
// plane zero-extended at its end), and stores only that corner of its
// results.  Hs = H and Ws = W: the planes as they are.
struct Rag {
    int Hs, Ws;
};

// Whole-plane path: every (b, c) plane is staged in LDS in one piece.
// Returns true if this build holds kernels for the shape.
bool plane_supported(const wtconv_shape& s);
// Workspace bytes the whole-plane weight-gradient kernels need.
size_t plane_workspace_bytes(const wtconv_shape& s);
// flip = false: forward (y = op(x)); flip = true: input gradient
// (dx = op^T(dy): 180-degree rotated kernels, no bias).
// `rg`: the stored planes (see Rag; {s.H, s.W} for planes of the kernel's
// own size).
hipError_t plane_apply(const wtconv_shape& s, const void* in,
                       const Params& p, void* out, bool flip,
                       hipStream_t stream, Rag rg);
hipError_t plane_bwd_weight(const wtconv_shape& s, const void* x,
                            const void* dy, const Params& p, const Grads& g,
                            void* workspace, hipStream_t stream, Rag rg);
// Input gradient and parameter gradients in one pass over x and dy.
hipError_t plane_bwd(const wtconv_shape& s, const void* x, const void* dy, const Params& p,
                     void* dx, const Grads& g, void* workspace, hipStream_t stream, Rag rg);
// Zero parameter gradients (empty batch or empty planes).
hipError_t zero_grads(const wtconv_shape& s, const Params& p, const Grads& g,
                      hipStream_t stream);
// Sum `rows` fp32 partial rows per channel in order and apply the chain rule
// through the fold (rows = 0 gives zero gradients).
hipError_t finalize_grads(const wtconv_shape& s, const float* part, int rows, const Params& p,
                          const Grads& g, hipStream_t stream);

// Tile path for planes too large for one workgroup's LDS: base conv and up to
// three levels per 32 x 32 output tile, deeper levels per plane.
bool tile_supported(const wtconv_shape& s);
size_t tile_workspace_bytes(const wtconv_shape& s);
hipError_t tile_apply(const wtconv_shape& s, const void* in, const Params& p, void* out,
                      bool flip, void* workspace, hipStream_t stream);
hipError_t tile_bwd_weight(const wtconv_shape& s, const void* x, const void* dy,
                           const Params& p, const Grads& g, void* workspace,
                           hipStream_t stream);
// Both gradients from one pass over the tiles of x and dy (with deeper
// levels: their input gradient from the box sums of dy before the pass,
// their weight taps after it).
hipError_t tile_bwd(const wtconv_shape& s, const void* x, const void* dy, const Params& p,
                    void* dx, const Grads& g, void* workspace, hipStream_t stream);

// Raise `fn`'s dynamic-LDS limit to `lds` where that exceeds 64 KiB (once
// per device and kernel).
hipError_t prepare_lds(const void* fn, size_t lds);
// Workgroups of `fn` (nt threads, lds bytes of dynamic LDS) that fit the
// current device at once: compute units times resident workgroups per unit,
// 1024 when it cannot be queried.  Queried once per device, kernel and size.
int resident_wgs(const void* fn, int nt, size_t lds);

// Planes of Hs x Ws -> planes of Hd x Wd: the top-left min(Hs,Hd) x
// min(Ws,Wd) corner copied, zeros elsewhere (zero extension or cropping).
hipError_t copy_planes(const void* src, void* dst, long planes, int Hs, int Ws, int Hd, int Wd,
                       int dtype, hipStream_t stream);

}  // namespace wtc
