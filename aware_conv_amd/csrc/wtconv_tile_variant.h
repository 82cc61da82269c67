// Host-side description of one instantiated tile-kernel family (large planes:
// TH x TW output tiles, the base conv and LT levels per tile).
#pragma once

#include "wtconv_kernels.h"

namespace wtc {

struct TileVariant {
    int K, LT, dtype;
    int TH, TW;    // tiles of the weight-gradient and fused backward kernels
    int ATH, ATW;  // tiles of the forward and input-gradient kernels
    int NT;
    const void* fwd;
    const void* bwi;
    const void* bww;
    const void* bwd;  // fused backward: input gradient and weight partials
    size_t lds_apply, lds_bww, lds_bwd;
};

// Tiles are 32 x 32 for the kernels that stage x and dy side by side; the
// forward and input gradient stage one tensor and take 32 x 64 tiles (less
// halo per output, fuller register tiles) where two workgroups still fit a
// compute unit's LDS, i.e. for k <= 5.
constexpr int kTileH = 32, kTileW = 32, kTileNT = 256;
constexpr int apply_tile_w(int k) { return k <= 5 ? 64 : 32; }

template <int K, int LT, typename T>
TileVariant make_tile_variant(int dtype) {
    constexpr int ATW = apply_tile_w(K);
    using G = dev::Geo<K, LT, kTileH, kTileW, 1, kTileNT, LT>;
    using GA = dev::Geo<K, LT, kTileH, ATW, 1, kTileNT, LT>;
    return TileVariant{
        K, LT, dtype, kTileH, kTileW, kTileH, ATW, kTileNT,
        reinterpret_cast<const void*>(&dev::k_tile_apply<K, LT, kTileH, ATW, kTileNT, T, false>),
        reinterpret_cast<const void*>(&dev::k_tile_apply<K, LT, kTileH, ATW, kTileNT, T, true>),
        reinterpret_cast<const void*>(&dev::k_tile_bww<K, LT, kTileH, kTileW, kTileNT, T>),
        reinterpret_cast<const void*>(&dev::k_tile_bwd1<K, LT, kTileH, kTileW, kTileNT, T>),
        dev::apply_lds_bytes<GA>(), dev::bww_lds_bytes<G>(), dev::tile_bwd1_lds_bytes<G>()};
}

// Tables of the per-k translation units (LT = 1, 2, 3; fp32 and fp16).
const TileVariant* tile_table_k1(int* n);
const TileVariant* tile_table_k3(int* n);
const TileVariant* tile_table_k5(int* n);
const TileVariant* tile_table_k7(int* n);

}  // namespace wtc
