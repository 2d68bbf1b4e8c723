// w4_config.cpp -- run-time dispatch configuration: environment, the tile
// table (parsed and validated as a whole), the dispatch log.
#include "w4_config.h"

#include <cerrno>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <set>
#include <sstream>

namespace w4 {

namespace {

std::mutex g_mu;
std::shared_ptr<const Config> g_cfg;
std::set<std::string> g_logged;

bool parse_int(const std::string& s, long lo, long hi, int& out) {
    if (s.empty()) return false;
    errno = 0;
    char* end = nullptr;
    const long v = strtol(s.c_str(), &end, 10);
    if (errno != 0 || !end || *end != '\0' || v < lo || v > hi) return false;
    out = (int)v;
    return true;
}

unsigned parse_force(const char* e, std::string& bad) {
    static const struct { const char* name; unsigned bit; } kNames[] = {
        {"gemv_generic", kForceGemvGeneric}, {"gemv_tiled", kForceGemvTiled},
        {"gemv_contig", kForceGemvContig},   {"smallm_valu", kForceSmallmValu},
        {"prefill_regs", kForcePrefillRegs}, {"i8_regs", kForceI8Regs},
        {"ordered_inline", kForceOrderedInline}, {"no_splitk", kForceNoSplitK}};
    unsigned f = 0;
    std::stringstream ss(e);
    std::string tok;
    while (std::getline(ss, tok, ',')) {
        if (tok.empty()) continue;
        bool found = false;
        for (const auto& n : kNames)
            if (tok == n.name) {
                f |= n.bit;
                found = true;
            }
        if (!found) bad = tok;
    }
    return f;
}

int env_index(const char* name, int lo, int hi) {
    const char* e = getenv(name);
    int v;
    if (e && parse_int(e, lo, hi, v)) return v;
    return -1;
}

std::shared_ptr<Config> from_env() {
    auto c = std::make_shared<Config>();
    const char* lg = getenv("W4_LOG");
    c->log = lg && *lg && strcmp(lg, "0") != 0;
    if (const char* e = getenv("W4_FORCE_PATH")) {
        std::string bad;
        c->force = parse_force(e, bad);
        if (!bad.empty()) {
            c->status = W4_ERR_ARG;
            c->error = "W4_FORCE_PATH: unknown path '" + bad + "'";
        }
    }
    c->prefill_cfg = env_index("W4_PREFILL_CFG", 0, 63);
    c->mfma_cfg = env_index("W4_MFMA_CFG", 0, 63);
    c->i8_ring = env_index("W4_I8_RING", 1, 63);
    if (const char* e = getenv("W4_SWEEP_POLL_LIMIT")) {
        int v;
        if (parse_int(e, 0, 1 << 30, v)) c->sweep_poll_limit = v;
    }
    if (const char* e = getenv("W4_I8_TILE")) {
        int mf = 0, nf = 0;
        if (sscanf(e, "%d,%d", &mf, &nf) == 2 && (mf == 2 || mf == 4) && (nf == 2 || nf == 4)) {
            c->i8_mf = mf;
            c->i8_nf = nf;
        }
    }
    if (const char* p = getenv("W4_TILE_TABLE")) {
        if (*p) {
            std::ifstream f(p, std::ios::binary);
            std::string text;
            if (f) {
                std::stringstream b;
                b << f.rdbuf();
                text = b.str();
            }
            std::string err;
            const int st = !f ? (err = std::string(p) + ": cannot be read", W4_ERR_ARG)
                              : parse_tile_table(text, p, c->table, err);
            if (st != W4_OK && c->status == W4_OK) {
                c->status = st;
                c->error = "W4_TILE_TABLE: " + err;
                c->table.clear();
            } else if (st == W4_OK) {
                c->table_source = p;
            }
        }
    }
    return c;
}

void install(std::shared_ptr<const Config> c) {
    g_cfg = std::move(c);
    g_logged.clear();
}

}  // namespace

int parse_tile_table(const std::string& text, const std::string& source,
                     std::vector<TileEntry>& out, std::string& err) {
    out.clear();
    if (text.size() > (1u << 20)) {
        err = source + ": larger than 1 MiB";
        return W4_ERR_ARG;
    }
    std::stringstream lines(text);
    std::string line;
    int ln = 0;
    auto bad = [&](int st, const std::string& why) {
        err = source + ":" + std::to_string(ln) + ": " + why;
        out.clear();
        return st;
    };
    while (std::getline(lines, line)) {
        ++ln;
        const size_t hash = line.find('#');
        if (hash != std::string::npos) line.resize(hash);
        std::stringstream ws(line);
        std::vector<std::string> tok;
        std::string t;
        while (ws >> t) tok.push_back(t);
        if (tok.empty()) continue;
        if (tok[0] != "gemv") return bad(W4_ERR_ARG, "unknown entry '" + tok[0] + "'");
        if (tok.size() != 10)
            return bad(W4_ERR_ARG, "a gemv entry has 10 fields: gemv N K group L U waves "
                                   "grid stages contig");
        int v[9];
        for (int i = 0; i < 9; ++i)
            if (!parse_int(tok[i + 1], INT_MIN, INT_MAX, v[i]))
                return bad(W4_ERR_ARG, "field " + std::to_string(i + 2) + " is not an integer");
        TileEntry e;
        e.N = v[0];
        e.K = v[1];
        e.group = v[2];
        GemvTile& g = e.t;
        g.L = v[3];
        g.U = v[4];
        g.waves = v[5];
        g.grid = v[6];
        g.stages = v[7];
        g.contig = v[8] == 1;
        if (e.group != 32 && e.group != 256 && e.group != 512)
            return bad(W4_ERR_SHAPE, "group must be 32, 256 or 512");
        if (e.N < 1 || e.N > kMaxN) return bad(W4_ERR_SHAPE, "N out of range");
        if (e.K < e.group || e.K > kMaxK || e.K % e.group != 0)
            return bad(W4_ERR_SHAPE, "K must be a positive multiple of group");
        if (g.L != 8 && g.L != 16 && g.L != 32 && g.L != 64)
            return bad(W4_ERR_SHAPE, "L must be 8, 16, 32 or 64");
        const int C = e.K / 32;
        if (g.U == 0) {
            g.generic = true;
        } else {
            if (g.U < 1 || g.U > kMaxU) return bad(W4_ERR_SHAPE, "U must be 0 (generic) or 1..8");
            if (g.U != (C + g.L - 1) / g.L)
                return bad(W4_ERR_SHAPE, "U must be ceil(K / 32 / L) = " +
                                             std::to_string((C + g.L - 1) / g.L));
            if ((e.K / e.group) & 1)
                return bad(W4_ERR_SHAPE, "the tiled loop needs an even number of groups per row");
        }
        if (g.waves < 1 || g.waves > 4) return bad(W4_ERR_SHAPE, "waves must be 1..4");
        if (g.grid < 0 || g.grid > 65535) return bad(W4_ERR_SHAPE, "grid must be 0 (auto) .. 65535");
        if (g.stages != 2 && g.stages != 3) return bad(W4_ERR_SHAPE, "stages must be 2 or 3");
        if (g.stages == 3 && (g.U < 1 || g.U > 4))
            return bad(W4_ERR_SHAPE, "three stages need a tiled loop with U <= 4");
        if (v[8] != 0 && v[8] != 1) return bad(W4_ERR_SHAPE, "contig must be 0 or 1");
        if (g.contig && (g.L < 16 || g.U < 1 || g.U > 3 || g.L * g.U != C || g.waves != 4))
            return bad(W4_ERR_SHAPE, "contig needs L >= 16, L U = K / 32, U <= 3 and 4 waves");
        for (const TileEntry& o : out)
            if (o.N == e.N && o.K == e.K && o.group == e.group)
                return bad(W4_ERR_ARG, "shape listed twice");
        if (out.size() >= 4096) return bad(W4_ERR_ARG, "more than 4096 entries");
        out.push_back(e);
    }
    return W4_OK;
}

std::shared_ptr<const Config> config() {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_cfg) install(from_env());
    return g_cfg;
}

int config_status() {
    const auto c = config();
    if (c->status != W4_OK) return fail(c->status, "%s", c->error.c_str());
    return W4_OK;
}

int reload_config() {
    auto c = from_env();
    const int st = c->status;
    const std::string msg = c->error;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        install(std::move(c));
    }
    if (st != W4_OK) return fail(st, "%s", msg.c_str());
    return W4_OK;
}

int load_tile_table(const char* path) {
    std::vector<TileEntry> table;
    std::string source;
    if (path) {
        std::ifstream f(path, std::ios::binary);
        if (!f) return fail(W4_ERR_ARG, "%s: cannot be read", path);
        std::stringstream b;
        b << f.rdbuf();
        std::string err;
        const int st = parse_tile_table(b.str(), path, table, err);
        if (st != W4_OK) return fail(st, "%s", err.c_str());
        source = path;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    auto c = std::make_shared<Config>(g_cfg ? *g_cfg : *from_env());
    c->table = std::move(table);
    c->table_source = source;
    if (c->error.rfind("W4_TILE_TABLE", 0) == 0) {
        c->status = W4_OK;
        c->error.clear();
    }
    install(std::move(c));
    return W4_OK;
}

bool table_tile(const Config& c, int N, int K, int group, GemvTile& t) {
    for (const TileEntry& e : c.table)
        if (e.N == N && e.K == K && e.group == group) {
            t = e.t;
            return true;
        }
    return false;
}

void log_dispatch(const Config& c, const std::string& what) {
    if (!c.log) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_logged.insert(what).second) return;
    fprintf(stderr, "w4a16: %s\n", what.c_str());
    fflush(stderr);
}

}  // namespace w4
