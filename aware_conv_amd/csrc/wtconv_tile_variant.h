// Host-side description of one instantiated tile-kernel family (large planes:
// TH x TW output tiles, the base conv and LT levels per tile).
#pragma once

#include "wtconv_kernels.h"

namespace wtc {

struct TileVariant {
    int K, LT, dtype;
    int TH, TW;    // tiles of the weight-gradient kernel
    int ATH, ATW;  // tiles of the forward and input-gradient kernels
    int BTW;       // tile width of the fused backward (height TH)
    int NT;
    const void* fwd;
    const void* bwi;
    const void* bww;
    const void* bwd;  // fused backward: input gradient and weight partials
    size_t lds_apply, lds_bww, lds_bwd;
};

// Tiles are 32 x 32 for the weight-gradient kernel, which stages x and dy
// side by side; the forward, input gradient and fused backward stage one
// tensor at a time and take 32 x 64 tiles (less halo per output, fuller
// register tiles) where two workgroups still fit a compute unit's LDS, i.e.
// for k <= 5.
constexpr int kTileH = 32, kTileW = 32, kTileNT = 256;
constexpr int apply_tile_w(int k) { return k <= 5 ? 64 : 32; }
// The fused backward (one LDS side) too: 32 x 64 tiles (20 outputs per lane,
// a 3x footprint for dy) fit two workgroups per unit at k <= 5 and beat
// three of 32 x 32 (12 outputs per lane, 4x): 512^2 backward 1053 -> 1027 us,
// 1024^2 4510 -> 4291 us.
constexpr int bwd_tile_w(int k) { return k <= 5 ? 64 : 32; }

template <int K, int LT, typename T>
TileVariant make_tile_variant(int dtype) {
    constexpr int ATW = apply_tile_w(K), BTW = bwd_tile_w(K);
    using G = dev::Geo<K, LT, kTileH, kTileW, 1, kTileNT, LT>;
    using GA = dev::GeoTileTrim<K, LT, kTileH, ATW, kTileNT>;
    using GB = dev::GeoTileTrim<K, LT, kTileH, BTW, kTileNT>;
    return TileVariant{
        K, LT, dtype, kTileH, kTileW, kTileH, ATW, BTW, kTileNT,
        reinterpret_cast<const void*>(&dev::k_tile_apply<K, LT, kTileH, ATW, kTileNT, T, false>),
        reinterpret_cast<const void*>(&dev::k_tile_apply<K, LT, kTileH, ATW, kTileNT, T, true>),
        reinterpret_cast<const void*>(&dev::k_tile_bww<K, LT, kTileH, kTileW, kTileNT, T>),
        reinterpret_cast<const void*>(&dev::k_tile_bwd1<K, LT, kTileH, BTW, kTileNT, T>),
        dev::apply_lds_bytes<GA>(), dev::bww_lds_bytes<G>(), dev::tile_bwd1_lds_bytes<GB>()};
}

// Tables of the per-k translation units (LT = 1, 2, 3; fp32 and fp16).
const TileVariant* tile_table_k1(int* n);
const TileVariant* tile_table_k3(int* n);
const TileVariant* tile_table_k5(int* n);
const TileVariant* tile_table_k7(int* n);

}  // namespace wtc
