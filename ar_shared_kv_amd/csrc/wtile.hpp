// The packed weight layout shared by the projections (layers.hip) and the LM
// head (lmhead.hip): tiles of 128 rows x 64 bf16 columns (16 KiB), the tiles
// of one 128-row block in column order, block after block; element (n, k) of
// an N x Kin weight sits at
// ((n / 128) * (Kin / 64) + k / 64) * 8192 + (n % 128) * 64 + k % 64,
// and the rows of the last block past N are zero.
#pragma once

namespace orthrus {

constexpr int kWTileRows = 128;
constexpr int kWTileCols = 64;

}  // namespace orthrus
