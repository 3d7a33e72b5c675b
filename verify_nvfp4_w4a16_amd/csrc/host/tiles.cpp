// (N, K)-keyed tile table and its default rule.  See tiles.h.
#include "tiles.h"

#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <map>
#include <mutex>
#include <sstream>
#include <utility>
#include <vector>

#include "nvfp4_w4a16.h"

namespace nvfp4 {
namespace {

using Key = std::pair<int64_t, int64_t>;

Tile default_tile(int64_t n, int64_t k);

// Built-in entries chosen by sweeping launch settings on MI355X (every
// kernel at M = 1, 2, 8, 16, 32 over cold weights; the segment count and
// grouping that gave the lowest times over those row counts).  Every entry's
// bits are the same at every row count; entries differ from the default rule
// only in waves and split (which set the bits) and mwaves (which does not).
const std::map<Key, Tile>& builtin_table() {
    static const std::map<Key, Tile> table = [] {
        std::map<Key, Tile> t;
        auto add = [&](int64_t n, int64_t k, int waves, int split, int mwaves) {
            Tile x = default_tile(n, k);
            x.waves = waves;
            x.split = split;
            x.mwaves = mwaves;
            t[{n, k}] = x;
        };
        add(8192, 4096, 8, 4, 0);      // q/o-sized products of the decode round
        add(4096, 8192, 8, 4, 4);      // 64 columns per many-row workgroup at every row count
        add(24576, 4096, 4, 1, 6);     // gate/up: 96 columns per many-row workgroup, one per CU
        add(4096, 12288, 8, 4, 4);     // down
        // the row-invariance and fused-QKV configurations (M = 1..32): 7 %
        // (M = 16) and 20-22 % (M = 17..32) faster than the default rule's
        // split 8 / split 4 with eight wavefronts above 16 rows, level at M <= 8
        add(4096, 4096, 8, 4, 4);
        add(12288, 4096, 8, 2, 8);
        return t;
    }();
    return table;
}

std::map<Key, Tile>& override_table() {
    static std::map<Key, Tile> table;
    return table;
}

// Default: one 16-column tile per wavefront; K cut into at most 8 segments
// of whole 128-k blocks (a function of K alone); up to four blocks per
// pipeline step; segment groups by default_split.
Tile default_tile(int64_t n, int64_t k) {
    Tile t;
    t.cols = 16;
    int64_t blocks = k / 128;
    int waves = 8;
    while (waves > 1 && blocks % waves != 0) waves /= 2;
    t.waves = waves;
    int64_t per = blocks / waves;
    t.unroll = per % 4 == 0 ? 4 : per % 2 == 0 ? 2 : 1;
    t.split = default_split(n, waves);
    t.mwaves = 0;
    return t;
}

}  // namespace

int default_split(int64_t n, int waves) {
    const int64_t groups = (n + 127) / 128;
    int split = 1;
    while (split < waves && groups * split < 256) split *= 2;
    return split;
}

bool tile_valid(const Tile& t, int64_t /*n*/, int64_t k) {
    if (t.cols != 16 && t.cols != 32 && t.cols != 64) return false;
    if (t.waves < 1 || t.waves > 8) return false;
    if (t.unroll != 1 && t.unroll != 2 && t.unroll != 4) return false;
    if (k % (int64_t(128) * t.unroll * t.waves) != 0) return false;
    if (t.split != 1 && t.split != 2 && t.split != 4 && t.split != 8) return false;
    if (t.split > t.waves || t.waves % t.split != 0) return false;
    if (t.mwaves != 0 && t.mwaves != 4 && t.mwaves != 6 && t.mwaves != 8) return false;
    return true;
}

Tile tile_for(int64_t n, int64_t k) {
    Key key{n, k};
    auto& ov = override_table();
    auto it = ov.find(key);
    if (it != ov.end()) return it->second;
    auto& bt = builtin_table();
    auto jt = bt.find(key);
    if (jt != bt.end() && tile_valid(jt->second, n, k)) return jt->second;
    return default_tile(n, k);
}

static int read_override_file() {
    const char* path = std::getenv("NVFP4_TILES");
    if (!path || !*path) return NVFP4_OK;
    std::ifstream in(path);
    if (!in) return NVFP4_ERR_TILEFILE;
    std::map<Key, Tile> table;
    std::string line;
    while (std::getline(in, line)) {
        auto hash = line.find('#');
        if (hash != std::string::npos) line.resize(hash);
        std::istringstream ss(line);
        // N K cols waves unroll [split [mwaves]], integers only
        std::vector<int64_t> v;
        std::string tok;
        while (ss >> tok) {
            char* endp = nullptr;
            const long long x = std::strtoll(tok.c_str(), &endp, 10);
            if (endp == tok.c_str() || *endp != '\0') return NVFP4_ERR_TILEFILE;
            v.push_back(x);
        }
        if (v.empty()) continue;                        // blank line
        if (v.size() < 5 || v.size() > 7) return NVFP4_ERR_TILEFILE;
        const int64_t n = v[0], k = v[1];
        for (size_t i = 2; i < v.size(); ++i)
            if (v[i] < 0 || v[i] > 64) return NVFP4_ERR_TILEFILE;
        Tile t;
        t.cols = static_cast<int>(v[2]);
        t.waves = static_cast<int>(v[3]);
        t.unroll = static_cast<int>(v[4]);
        t.split = v.size() > 5 ? static_cast<int>(v[5]) : 1;
        t.mwaves = v.size() > 6 ? static_cast<int>(v[6]) : 0;
        if (nvfp4_linear_shape_ok(1, n, k) != NVFP4_OK || !tile_valid(t, n, k))
            return NVFP4_ERR_TILEFILE;
        table[{n, k}] = t;
    }
    override_table() = std::move(table);
    return NVFP4_OK;
}

int load_tile_override() {
    static std::once_flag once;
    static int status = NVFP4_OK;
    std::call_once(once, [] { status = read_override_file(); });
    return status;
}

std::string tile_text(int64_t n, int64_t k, const Tile& t) {
    char buf[320];
    int64_t groups = (n + t.cols - 1) / t.cols;
    std::snprintf(buf, sizeof buf,
                  "N=%lld K=%lld cols=%d waves=%d unroll=%d split=%d mwaves=%d k_per_wave=%lld "
                  "grid=%lld block=%d",
                  (long long)n, (long long)k, t.cols, t.waves, t.unroll, t.split, t.mwaves,
                  (long long)(k / t.waves), (long long)groups, 64 * t.waves);
    return buf;
}

}  // namespace nvfp4
