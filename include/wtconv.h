/*
 * wtconv.h -- C ABI of the fused WTConv layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer (a multi-level 2-D Haar wavelet depthwise convolution, the WTConv
 * operator of "Fast and Memory-Efficient Wavelet Convolutions via I/O-Aware
 * Reformulation", Aflalo et al., arXiv 2608.10805) is a drop-in replacement
 * for a depthwise convolution: same NCHW tensor in and out, per-channel
 * learned scales.  Per channel c and image b, with X the H x W plane:
 *
 *   A^0 = X;  for l = 1..L: (S_LL, S_LH, S_HL, S_HH)^l = H(A^{l-1}), A^l = S^l_LL
 *   Y^l_s = s_wav[l,c,s] * conv_{w_wav[l,c,s]}(S^l_s)
 *   R^{L+1} = 0;  for l = L..1: R^l = H^T(Y^l_LL + R^{l+1}, Y^l_LH, Y^l_HL, Y^l_HH)
 *   y = s_base[c] * (conv_{w_base[c]}(X) + b_base[c]) + R^1
 *
 * H is the stride-2 2x2 orthonormal Haar analysis with taps +-1/2 (rows index
 * y, columns x): LL = 1/2[[1,1],[1,1]], LH = 1/2[[1,-1],[1,-1]],
 * HL = 1/2[[1,1],[-1,-1]], HH = 1/2[[1,-1],[-1,1]] (the filter matrices of
 * the cybasar.com WTConv tutorial, section 3); H^T is its transpose.  conv is
 * a k x k cross-correlation with 'same' zero padding, each level zero-padding
 * its own coefficient grid.  The pipeline of the reference implementation
 * (one op per stage, every intermediate through device memory) and the
 * three reformulations computed here instead -- Haar analysis recomputed on
 * chip, single-pass synthesis indexed by output-coordinate bits, learned
 * scales folded into the filters -- are described in the gist.science/pt
 * summary, "Resumo Tecnico", section "Metodologia".  Results equal the
 * unfused operator up to floating-point evaluation order ("Principais
 * Contribuicoes").
 *
 * Sides of any length: a grid with an odd side gets one zero row (column)
 * appended at its end before its analysis, as the stride-2 'SAME' Haar
 * convolutions of the cybasar.com tutorial (section 3) do, and the synthesis
 * crops back to that grid.  The library runs such shapes on planes
 * zero-extended at their end to a multiple of 2^L and crops the results,
 * which is the same operator: the whole-plane kernels read each stored plane
 * as the corner of the extended one (zeros beyond it) and write only that
 * corner back; the tile kernels run on zero-extended copies in the
 * workspace.
 *
 * Tensors (all contiguous, row-major, device memory, element type `dtype`):
 *   x, y, dy, dx : [B][C][H][W]
 *   w_base       : [C][1][k][k]       b_base, s_base : [C]
 *   w_wav        : [L][C][4][k][k]    s_wav          : [L][C][4]
 *   subband order (LL, LH, HL, HH).
 *
 * The library sees pointers only: each must address at least the elements
 * its shape implies, on the current HIP device; a shorter buffer, or host
 * memory, is read or written out of bounds on the GPU.
 *
 * Arithmetic: loads are widened to fp32, every sum is accumulated in fp32
 * (the parameter gradients' partial rows are then summed, and put through
 * the chain rule of the scale folding, in fp64) and each output is rounded
 * once (round-to-nearest-even) to `dtype`.
 *
 * Ownership and threading: the caller owns every buffer, the workspace
 * included; the workspace may not overlap any other buffer of the call
 * (WTCONV_ERR_ALIAS).  The library never allocates, frees or synchronises; every call
 * only enqueues kernels on `stream` (a hipStream_t, NULL for the default
 * stream) and returns.  The library keeps no state between calls, apart
 * from the static scratch of wtconv_bwd_noalloc (see there).
 *
 * Errors: every argument check happens before anything is enqueued, so a
 * negative return means nothing ran.  WTCONV_ERR_HIP means a launch failed
 * (hipGetLastError); the outputs are then undefined.
 */
#ifndef WTCONV_H
#define WTCONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { WTCONV_F32 = 0, WTCONV_F16 = 1 } wtconv_dtype;

typedef struct {
    int B, C, H, W; /* batch, channels, height, width (NCHW) */
    int L;          /* Haar levels, 1 <= L <= WTCONV_MAX_LEVELS */
    int k;          /* odd depthwise kernel size, 1 <= k <= 7 */
    int dtype;      /* wtconv_dtype of every tensor, parameters included */
} wtconv_shape;

#define WTCONV_MAX_LEVELS 6

#define WTCONV_OK 0
#define WTCONV_ERR_NULL (-1)        /* a required pointer is NULL */
#define WTCONV_ERR_SHAPE (-2)       /* negative or too large dimension */
#define WTCONV_ERR_KERNEL (-3)      /* k even, < 1 or > 7 */
#define WTCONV_ERR_LEVELS (-4)      /* L outside 1..WTCONV_MAX_LEVELS */
#define WTCONV_ERR_DTYPE (-5)       /* dtype not a wtconv_dtype */
#define WTCONV_ERR_ALIGN (-6)       /* activation/workspace pointer not 16-byte aligned,
                                       or parameter pointer not element aligned */
#define WTCONV_ERR_WORKSPACE (-7)   /* ws_bytes below wtconv_workspace_size() */
#define WTCONV_ERR_UNSUPPORTED (-8) /* valid shape this build has no kernel for
                                       (a plane of 2^31 bytes or more) */
#define WTCONV_ERR_ALIAS (-9)       /* an output overlaps an input or another output, or
                                       the workspace overlaps any buffer of the call */
#define WTCONV_ERR_SCRATCH (-10)    /* wtconv_bwd_noalloc: the shape needs more workspace
                                       than WTCONV_NOALLOC_SCRATCH_BYTES */
#define WTCONV_ERR_HIP (-100)       /* a kernel launch failed */

/*
 * Bytes of device workspace the calls below need for shape `s` (the maximum
 * over every call below); 0 is possible.
 * Returns WTCONV_OK or a shape error; *bytes is set only on success.
 */
int wtconv_workspace_size(const wtconv_shape* s, size_t* bytes);

/*
 * Forward: y = WTConv(x) as defined above (gist.science/pt, "Metodologia":
 * fused Haar analysis, closed-form synthesis, folded scales).  x and y are
 * [B][C][H][W]; y must not overlap x.  Planes too large for on-chip staging
 * with more than three levels use the workspace for the deeper levels (the
 * 8 x 8 box sums of the input, their contribution, and for the largest
 * planes their Haar levels: a few 1/64 of the input), and shapes run on
 * zero-extended tiled planes keep those planes there; pass wtconv_workspace_size()
 * bytes, or NULL when it reported 0.
 */
int wtconv_fwd(const wtconv_shape* s, const void* x, const void* w_base,
               const void* b_base, const void* s_base, const void* w_wav,
               const void* s_wav, void* y, void* workspace, size_t ws_bytes,
               void* stream);

/*
 * Input gradient: dx = (dy/dx)^T dy, the transpose of the layer's linear
 * part, which is the same operator with every kernel rotated by 180 degrees
 * and no bias (the gradient the paper verifies alongside the forward,
 * gist.science/pt "Principais Contribuicoes").  dy and dx are [B][C][H][W];
 * dx must not overlap dy.  b_base is not needed.  Workspace as for
 * wtconv_fwd.
 */
int wtconv_bwd_input(const wtconv_shape* s, const void* dy,
                     const void* w_base, const void* s_base,
                     const void* w_wav, const void* s_wav, void* dx,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * Parameter gradients of <dy, y(x)> ("all parameter gradients", same
 * passage): dw_base [C][1][k][k], db_base [C], ds_base [C],
 * dw_wav [L][C][4][k][k], ds_wav [L][C][4], in `dtype`.  Gradients are
 * overwritten, not accumulated; no gradient buffer may overlap x, dy, a
 * parameter or another gradient (WTCONV_ERR_ALIAS).  Sums over the batch and the plane are taken
 * in a fixed order, so results are bitwise reproducible for a given shape.
 * Needs wtconv_workspace_size() bytes of workspace.
 */
int wtconv_bwd_weight(const wtconv_shape* s, const void* x, const void* dy,
                      const void* w_base, const void* b_base,
                      const void* s_base, const void* w_wav,
                      const void* s_wav, void* dw_base, void* db_base,
                      void* ds_base, void* dw_wav, void* ds_wav,
                      void* workspace, size_t ws_bytes, void* stream);

/*
 * Fused backward: the results of wtconv_bwd_input and wtconv_bwd_weight from
 * one call that reads x and dy once (the training step's backward, whose
 * speed-up over the unfused layer gist.science/pt reports under
 * "Resultados").  Arguments are those of the two calls, dx included: dx
 * [B][C][H][W] must overlap neither x nor dy nor a parameter, nor a
 * gradient buffer; the gradients are overwritten.
 * Results equal the two separate calls up to floating-point evaluation
 * order, and the parameter gradients are bitwise reproducible for a given
 * shape.  Needs wtconv_workspace_size() bytes of workspace.
 */
int wtconv_bwd(const wtconv_shape* s, const void* x, const void* dy,
               const void* w_base, const void* b_base, const void* s_base,
               const void* w_wav, const void* s_wav, void* dx, void* dw_base,
               void* db_base, void* ds_base, void* dw_wav, void* ds_wav,
               void* workspace, size_t ws_bytes, void* stream);

/*
 * Allocation-free fused backward, for callers that cannot allocate device
 * memory or cannot own a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments and
 * results as wtconv_bwd without the workspace, which is instead a static
 * array of WTCONV_NOALLOC_SCRATCH_BYTES in device memory that every GPU the
 * library runs on holds until the process ends (its address is looked up
 * once per device, on the first call there).  Shapes whose
 * wtconv_workspace_size() exceeds that size are refused with
 * WTCONV_ERR_SCRATCH before anything runs (the WTConvNeXt stage shapes need
 * a few MiB, 8 x 64 x 512 x 512 at five levels about 33 MiB).  The call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library call.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap in
 * time on one GPU -- on different streams, or from different threads --
 * race on it and give undefined results; order them on one stream.
 */
#define WTCONV_NOALLOC_SCRATCH_BYTES (64u << 20)
int wtconv_bwd_noalloc(const wtconv_shape* s, const void* x, const void* dy,
                       const void* w_base, const void* b_base, const void* s_base,
                       const void* w_wav, const void* s_wav, void* dx,
                       void* dw_base, void* db_base, void* ds_base,
                       void* dw_wav, void* ds_wav, void* stream);

/* Static description of an error code (never NULL). */
const char* wtconv_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* WTCONV_H */
