/*
 * dwconv.h -- C ABI of a plain depthwise k x k convolution with bias for
 * AMD Instinct MI355X (gfx950): the layer WTConv replaces, kept as the
 * baseline the pages compare against (WTConv with k = 5 against a 7 x 7
 * depthwise convolution, in training and in inference: gist.science/pt,
 * "Resumo Tecnico", "Resultados"; insight.aitobox.com, "Performance
 * Evaluation").
 *
 *   y[b,c] = conv_{w[c]}(x[b,c]) + bias[c]
 *
 * conv is a k x k cross-correlation with 'same' zero padding (k odd).  It
 * runs on the same whole-plane kernels as the WTConv layer with no wavelet
 * levels, so the two are measured with the same machinery.
 *
 * Tensors (contiguous, row-major, device memory, element type `dtype`):
 *   x, y, dy, dx : [B][C][H][W]      w, dw : [C][1][k][k]      bias, db : [C]
 * Arithmetic, ownership, threading and error codes are those of wtconv.h:
 * fp32 accumulation, one rounding per output; the caller owns every buffer,
 * each of at least the elements its shape implies (pointers only are seen);
 * calls only enqueue on `stream`; every check happens before anything is
 * enqueued.  Shapes without a kernel in this build (the ConvNeXt-T stage
 * shapes at k = 7 are built) return WTCONV_ERR_UNSUPPORTED.
 */
#ifndef DWCONV_H
#define DWCONV_H

#include <stddef.h>

#include "wtconv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int B, C, H, W; /* batch, channels, height, width (NCHW) */
    int k;          /* odd kernel size, 1 <= k <= 7 */
    int dtype;      /* wtconv_dtype of every tensor */
} dwconv_shape;

/* Bytes of device workspace dwconv_bwd needs for shape `s`. */
int dwconv_workspace_size(const dwconv_shape* s, size_t* bytes);

/* y = conv_w(x) + bias.  y must not overlap x. */
int dwconv_fwd(const dwconv_shape* s, const void* x, const void* w,
               const void* bias, void* y, void* stream);

/*
 * Gradients of <dy, y(x)>: dx (the conv with the kernel rotated by 180
 * degrees), dw = sum over the batch and the plane of dy times shifted x, and
 * db = sum of dy; one pass over x and dy.  dx must overlap neither x nor dy;
 * dw and db are overwritten, summed in a fixed order (bitwise reproducible
 * for a given shape).  Needs dwconv_workspace_size() bytes of workspace.
 */
int dwconv_bwd(const dwconv_shape* s, const void* x, const void* dy,
               const void* w, void* dx, void* dw, void* db, void* workspace,
               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DWCONV_H */
