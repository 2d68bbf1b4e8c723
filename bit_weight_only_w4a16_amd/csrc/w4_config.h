// w4_config.h -- run-time dispatch configuration (internal): the per-shape
// GEMV tile table, forced kernel paths, tuning overrides and the dispatch log.
//
// Read from the environment once, on the first dispatch, and again on
// w4_config_reload(); W4_TILE_TABLE names a tile table file (format in
// include/w4a16.h), validated as a whole before use.
#pragma once

#include <memory>
#include <string>
#include <vector>

#include "w4_dispatch.h"

namespace w4 {

// W4_FORCE_PATH names (comma-separated), each forcing one kernel family
// wherever it applies.
enum ForcePath : unsigned {
    kForceGemvGeneric = 1u << 0,   // M = 1: the generic loop (chunks re-read per row)
    kForceGemvTiled = 1u << 1,     // M = 1: the register-tiled loop, heuristic tile
    kForceGemvContig = 1u << 2,    // M = 1: contiguous row ranges where the tile allows
    kForceSmallmValu = 1u << 3,    // small M: the vector-ALU kernel
    kForcePrefillRegs = 1u << 4,   // M > 16: the register-staged matrix-core kernel
    kForceI8Regs = 1u << 5,        // int8 twin: the register-staged kernel
    kForceOrderedInline = 1u << 6, // decode-ordered sweep: decode while multiplying
    kForceNoSplitK = 1u << 7,      // 2..64 rows: not the split-K matrix-core kernel
};

struct TileEntry {
    int N, K, group;
    GemvTile t;
};

struct Config {
    bool log = false;               // W4_LOG: print each distinct dispatch once
    unsigned force = 0;             // W4_FORCE_PATH
    int prefill_cfg = -1;           // W4_PREFILL_CFG: a prefill tiling index
    int mfma_cfg = -1;              // W4_MFMA_CFG: a register-staged tiling index
    int i8_ring = -1;               // W4_I8_RING: 1..4 a ring tiling (0 = W4_FORCE_PATH i8_regs)
    int i8_mf = 0, i8_nf = 0;       // W4_I8_TILE "MF,NF": register-staged int8 tile
    long sweep_poll_limit = -1;     // W4_SWEEP_POLL_LIMIT: completion polls per op (-1: default)
    std::vector<TileEntry> table;   // W4_TILE_TABLE or w4_tile_table_load
    std::string table_source;       // its path, "" for none
    int status = 0;                 // W4_OK, or why W4_TILE_TABLE could not be used
    std::string error;              // and the message
};

// The current configuration (loaded on first use).  The snapshot stays valid
// while the caller holds the pointer, across a concurrent reload.
std::shared_ptr<const Config> config();

// W4_OK, or the status (and last-error message) of a W4_TILE_TABLE that
// could not be used: every dispatching entry point returns it.
int config_status();

// Re-reads the environment (and W4_TILE_TABLE).
int reload_config();

// Parses a tile table; W4_OK or W4_ERR_ARG / W4_ERR_SHAPE with the line in
// `err`.  `source` names it in messages.
int parse_tile_table(const std::string& text, const std::string& source,
                     std::vector<TileEntry>& out, std::string& err);

// Replaces the table of the current configuration (path NULL: no table).
int load_tile_table(const char* path);

// The table's tile for a shape, if any.
bool table_tile(const Config& c, int N, int K, int group, GemvTile& t);

// Prints `what` once per distinct text when W4_LOG is set.
void log_dispatch(const Config& c, const std::string& what);

}  // namespace w4
