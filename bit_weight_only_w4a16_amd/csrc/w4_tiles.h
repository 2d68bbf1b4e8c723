// w4_tiles.h -- the built-in GEMV tile table (included by w4_gemv.hip).
// Written by `python -m bit_weight_only_w4a16_amd.tune --header` from
// tiles_mi355x.txt (searched on MI355X; the file's comments give
// the cold time of each entry and of the heuristic tile).
constexpr int kBuiltinTileCount = 6;
static const TileEntry kBuiltinTiles[6] = {
    {256, 512, 32, GemvTile{16, 1, 1, 0, 2, false, false}},
    {2560, 1536, 32, GemvTile{64, 1, 4, 0, 3, false, false}},
    {1536, 2048, 32, GemvTile{64, 1, 4, 256, 3, false, false}},
    {12288, 1536, 32, GemvTile{16, 3, 4, 256, 3, false, false}},
    {1536, 6144, 32, GemvTile{64, 3, 4, 256, 3, false, false}},
    {262144, 1536, 32, GemvTile{8, 6, 4, 256, 2, false, false}},
};
