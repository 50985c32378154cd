// Host-side tile table of libbfq: per (N, K, input dtype, block shape) a map from M bucket
// to a launch configuration, loaded from JSON, with nearest-M lookup.
//
// Page cited: "vLLM 量化 Kernel 配置机制：W8A8 Block FP8 Triton 内核的调优、选择与回退原理"
//   §1 (one tuned entry per shape x device x dtype x block shape), §2 (each entry maps a
//   non-uniform grid of M values to launch parameters), §4.1 (looked up once and cached;
//   a missing entry is not an error but a warning and a default config), §4.2 (the entry
//   whose M key is nearest to the runtime M is used).
#pragma once
#include <stdint.h>

#include <map>
#include <string>
#include <vector>

#include "../../include/bfq.h"

namespace bfq {

struct TableKey {
    int64_t N, K;
    int qtype;
    int wlayout;   // weight layout the tuned kernels read (W_ROW / W_PACKED16)
    int sfmt;      // scale handling the entry was tuned for (S_FP32 / S_UE8M0 / S_CHANNEL)
    int64_t E = 0; // expert count of a grouped (MoE) entry, 0 for a dense one ([CONFIG] §5)
    bool operator<(const TableKey& o) const {
        if (E != o.E) return E < o.E;
        if (N != o.N) return N < o.N;
        if (K != o.K) return K < o.K;
        if (qtype != o.qtype) return qtype < o.qtype;
        if (wlayout != o.wlayout) return wlayout < o.wlayout;
        return sfmt < o.sfmt;
    }
};

struct TileTable {
    std::map<TableKey, std::map<int64_t, bfq_tile>> entries;   // M bucket -> tile
};

// Parse a table file. On failure returns false and fills `err`.
bool parse_tile_table(const std::string& text, TileTable& out, std::string& err);

// Nearest bucket to M among the keys (ties to the smaller key; beyond the grid -> the end).
int64_t nearest_bucket(const std::map<int64_t, bfq_tile>& buckets, int64_t M);

}  // namespace bfq
