// Host side of libbfq: the C-ABI entry points of include/bfq.h — argument validation before
// any launch, tile selection (table + default rule), kernel dispatch and status reporting.
//
// Pages cited by title and section:
//   [BENCH]  "vLLM DeepGEMM FP8 Block GEMM 基准测试 ..." §4.1-§4.2 (operations, layouts,
//            preallocated output; the dispatch precondition of bf16 output, N a multiple of
//            64 and K a multiple of 128)
//   [CONFIG] "vLLM 量化 Kernel 配置机制 ..." §4.1-§4.2 (lookup, nearest M, warning + default)
//   [HELION] "Building a High-Performance and Portable vLLM Linear Backend with Helion",
//            scope section (per-token x per-channel scale formats), kernel section (swap-AB
//            below 32 tokens on Hopper; split-K for small M/N)
#include <dlfcn.h>

#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>

#include "bfq_internal.h"
#include "tile_table.h"

using namespace bfq;

// Workspace of the allocation-free GEMM entry point (bfq_block_gemm_noalloc, below).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_last_error;

bfq_status fail(bfq_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Largest output count (M * N, grouped: T * topk * N) the GEMMs take: 2^40 elements, far past
// any device memory, keeps split-K workspace sizes (256 splits of fp32) and the reduce
// kernel's one-dimensional grid within range.
constexpr int64_t kMaxOutputs = int64_t(1) << 40;

// a * b >= kMaxOutputs for positive a, b, without overflow
bool too_many_outputs(int64_t a, int64_t b) { return a > 0 && b > 0 && a > (kMaxOutputs - 1) / b; }

// ------------------------------------------------------------------ tile table ----
std::mutex g_table_mu;
TileTable g_table;
bool g_table_loaded = false;

std::string default_table_path() {
    const char* env = std::getenv("BFQ_TILE_TABLE");
    if (env && *env) return env;
    Dl_info info;
    if (dladdr((void*)&default_table_path, &info) && info.dli_fname) {
        std::string so = info.dli_fname;
        size_t slash = so.rfind('/');
        std::string dir = slash == std::string::npos ? "." : so.substr(0, slash);
        return dir + "/tables/gfx950.json";
    }
    return "tables/gfx950.json";
}

bool read_file(const std::string& path, std::string& text) {
    std::ifstream f(path, std::ios::binary);
    if (!f) return false;
    std::ostringstream ss;
    ss << f.rdbuf();
    text = ss.str();
    return true;
}

const KernelEntry* find_kernel(const bfq_tile& t, int qtype, int otype, int wlayout, int sfmt,
                               int moe = 0);

// Every table tile must name a compiled kernel; otherwise the table is rejected.
bool validate_table(const TileTable& t, std::string& err) {
    for (auto& e : t.entries)
        for (auto& b : e.second) {
            if (!find_kernel(b.second, e.first.qtype, O_BF16, e.first.wlayout, e.first.sfmt,
                             e.first.E > 0 ? 1 : 0)) {
                err = "table entry N=" + std::to_string(e.first.N) + " K=" +
                      std::to_string(e.first.K) + " M=" + std::to_string(b.first) +
                      " names a tile that is not compiled";
                return false;
            }
            if (b.second.split_k < 1 || b.second.split_k > 256 || b.second.group_m < 1 ||
                b.second.raster < 0 || b.second.raster > 1) {
                err = "table entry has split_k outside [1, 256], group_m < 1 or raster not 0/1";
                return false;
            }
        }
    return true;
}

bfq_status load_table_locked(const std::string& path, bool strict) {
    std::string text, err;
    TileTable t;
    if (!read_file(path, text)) {
        if (strict) return fail(BFQ_ERR_TABLE, "cannot read tile table '" + path + "'");
        g_table = TileTable{};
        g_table_loaded = true;
        return BFQ_OK;
    }
    if (!parse_tile_table(text, t, err) || !validate_table(t, err)) {
        if (strict) return fail(BFQ_ERR_TABLE, "tile table '" + path + "': " + err);
        g_table = TileTable{};
        g_table_loaded = true;
        return BFQ_OK;
    }
    g_table = std::move(t);
    g_table_loaded = true;
    return BFQ_OK;
}

void ensure_table() {
    std::lock_guard<std::mutex> lk(g_table_mu);
    if (!g_table_loaded) load_table_locked(default_table_path(), false);
}

// ------------------------------------------------------------------ registry ----
bool same_shape(const bfq_tile& a, const bfq_tile& b) {
    if (a.variant != b.variant || a.bm != b.bm || a.bn != b.bn || a.waves_m != b.waves_m ||
        a.waves_n != b.waves_n || a.stages != b.stages)
        return false;
    return a.sched == b.sched;
}

// A kernel serves scale format sfmt if it takes any fp32 block scales (S_FP32) or if the block
// scales are declared powers of two (a S_UE8M0 kernel applies them inside the MFMA);
// per-token x per-channel scales (S_CHANNEL) need a kernel built for them.
// Packed UE8M0 activation-scale words (S_PACKED): the swap-AB instances built for them, or any
// block-scale kernel of variants 0 and 2 (they read packed words through a runtime flag).
bool serves(const KernelEntry& k, int sfmt) {
    if (sfmt == S_CHANNEL || k.sfmt == S_CHANNEL) return k.sfmt == sfmt;
    if (sfmt == S_PACKED) return k.sfmt == S_PACKED || k.tile.variant != 1;
    if (k.sfmt == S_PACKED) return false;
    return k.sfmt == S_FP32 || sfmt == S_UE8M0;
}

// moe = 1: the grouped (MoE) kernels (variants 0 and 1)
const KernelEntry* find_kernel(const bfq_tile& t, int qtype, int otype, int wlayout, int sfmt,
                               int moe) {
    if (t.bk != 0 && t.bk != 128) return nullptr;
    int n = 0;
    const KernelEntry* list = nullptr;
    if (moe) list = t.variant == 0 ? moe_std_kernels(&n) : t.variant == 1 ? moe_swapab_kernels(&n) : nullptr;
    else list = t.variant == 0   ? std_kernels(&n)
                : t.variant == 1 ? swapab_kernels(&n)
                : t.variant == 2 ? streamk_kernels(&n)
                                 : nullptr;
    for (int i = 0; list && i < n; ++i)
        if (list[i].qtype == qtype && list[i].otype == otype && list[i].wlayout == wlayout &&
            list[i].moe == moe && serves(list[i], sfmt) && same_shape(list[i].tile, t))
            return &list[i];
    return nullptr;
}

constexpr int64_t kNumCUs = 256;   // MI355X: 8 XCDs x 32 CUs

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compiled-in default ([CONFIG] §4.1: no tuned entry -> a fixed default config). Below 32
// tokens the swap-AB streaming kernel ([HELION]: the Hopper rule dispatches swap-AB for
// M < 32), else the standard kernel with the largest tile that still yields one workgroup
// per CU, among the tiles compiled for this code type, weight layout and scale format (the
// int8 kernels, for one, have no 128x256 tile). Split-K is added until the grid covers the
// CUs, keeping >= 4 K blocks per split.
bfq_tile default_tile(int64_t M, int64_t N, int64_t K, int qtype, int wlayout, int sfmt) {
    const int64_t KB = K / 128;
    bfq_tile t{};
    t.bk = 128;
    t.split_k = 1;
    int64_t ctas;
    if (M < 32) {
        t.variant = 1;
        t.bm = M <= 16 ? 16 : 32;
        t.bn = 128;
        t.waves_m = 1;
        t.waves_n = 4;
        t.stages = 4;
        t.group_m = 1;
        ctas = ceil_div(N, t.bn) * ceil_div(M, t.bm);
    } else {
        static const int shapes[4][4] = {{256, 256, 4, 2}, {128, 256, 2, 2}, {128, 128, 2, 2}, {64, 128, 1, 2}};
        t.variant = 0;
        t.stages = 2;
        t.group_m = 8;
        // the shape's schedule: per-token x per-channel scales accumulate the whole K (sched 4);
        // power-of-two fp8 scales use the block-scaled MFMA (sched 3) where it is compiled;
        // otherwise the per-block FMA (sched 0)
        auto shaped = [&](int i) {
            bfq_tile s = t;
            s.bm = shapes[i][0];
            s.bn = shapes[i][1];
            s.waves_m = shapes[i][2];
            s.waves_n = shapes[i][3];
            s.sched = sfmt == S_CHANNEL ? 4 : 0;
            if (sfmt == S_UE8M0 && qtype == Q_FP8) {
                s.sched = 3;
                if (!find_kernel(s, qtype, O_BF16, wlayout, sfmt)) s.sched = 0;
            }
            return s;
        };
        int pick = -1, last = -1;
        for (int i = 0; i < 4; ++i) {
            if (!find_kernel(shaped(i), qtype, O_BF16, wlayout, sfmt)) continue;
            last = i;
            if (ceil_div(M, shapes[i][0]) * ceil_div(N, shapes[i][1]) >= kNumCUs) { pick = i; break; }
        }
        t = shaped(pick >= 0 ? pick : last >= 0 ? last : 3);
        ctas = ceil_div(M, t.bm) * ceil_div(N, t.bn);
    }
    while (ctas * t.split_k < kNumCUs && KB / (t.split_k * 2) >= 4) t.split_k *= 2;
    return t;
}

// Batch-invariant tiles ([CONFIG] §5): every output element is computed by one 16x16x128
// MFMA per K block (int8: two chained, exact) and fma(P, sa*sw, acc) in ascending block
// order, whatever the tile. Excluded: split-K, in-workgroup K splits and stream-K (they sum
// partial K ranges) and, with row-major weights, the swap-AB kernels (their token/weight
// fragments take a different K order inside the MFMA than the standard kernel's).
bfq_tile invariant_tile(int64_t M, int wlayout, int sfmt) {
    bfq_tile t{};
    t.bk = 128;
    t.split_k = 1;
    t.group_m = 8;
    t.stages = 2;
    t.waves_m = 1;
    if (wlayout == W_PACKED16 && M <= 128) {
        t.variant = 1;
        if (M <= 16) {              // per-wave tokens, 4 strips of 32 rows
            t.bm = 16; t.bn = 128; t.waves_n = 4; t.stages = 4; t.sched = 0;
        } else {                    // tokens shared through LDS, 8 strips of 16 rows
            t.bm = M <= 32 ? 32 : M <= 64 ? 64 : 128; t.bn = 128; t.waves_n = 8; t.stages = 4;
            t.sched = 1;
        }
        t.group_m = 1;
        return t;
    }
    t.variant = 0;
    t.sched = sfmt == S_CHANNEL ? 4 : 0;
    if (M <= 64) { t.bm = 64; t.bn = 128; t.waves_m = 1; t.waves_n = 2; }
    else if (M <= 512) { t.bm = 128; t.bn = 128; t.waves_m = 2; t.waves_n = 2; }
    else { t.bm = 256; t.bn = 256; t.waves_m = 4; t.waves_n = 2; }
    return t;
}

int g_batch_invariant = -1;   // -1: not yet read from the environment

bool batch_invariant() {
    if (g_batch_invariant < 0) {
        const char* e = std::getenv("BFQ_BATCH_INVARIANT");
        g_batch_invariant = (e && e[0] == '1') ? 1 : 0;
    }
    return g_batch_invariant == 1;
}

// Grouped (MoE) default: the tile follows the average rows per active expert, r = pairs /
// min(E, pairs) (a stand-in for the per-expert M): streaming swap-AB up to 128 rows (each
// expert's weights are read once; tokens per wave up to 16, shared through LDS above), then
// standard tiles. No split-K: E experts x N strips already fill the device.
bfq_tile moe_default_tile(int64_t T, int64_t topk, int64_t E, int sfmt) {
    const int64_t pairs = T * topk, active = E < pairs ? E : pairs;
    const int64_t r = active > 0 ? (pairs + active - 1) / active : 1;
    bfq_tile t{};
    t.bk = 128;
    t.split_k = 1;
    t.group_m = 1;
    if (r <= 16) {
        t.variant = 1; t.bm = 16; t.bn = 128; t.waves_m = 1; t.waves_n = 4; t.stages = 4; t.sched = 0;
    } else if (r <= 128) {
        t.variant = 1; t.bm = r <= 32 ? 32 : r <= 64 ? 64 : 128; t.bn = 128; t.waves_m = 1;
        t.waves_n = 8; t.stages = 4; t.sched = 1;
    } else {
        t.variant = 0; t.stages = 2;
        t.sched = (sfmt == S_UE8M0) ? 3 : 0;
        if (r <= 256) { t.bm = 128; t.bn = 128; t.waves_m = 2; t.waves_n = 2; }
        else if (t.sched == 3) { t.bm = 256; t.bn = 256; t.waves_m = 4; t.waves_n = 2; }
        else { t.bm = 128; t.bn = 256; t.waves_m = 2; t.waves_n = 2; }
    }
    return t;
}

int qtype_of(bfq_dtype d) { return d == BFQ_E4M3FN ? Q_FP8 : Q_INT8; }

int otype_of(bfq_dtype d) { return d == BFQ_BF16 ? O_BF16 : d == BFQ_FP16 ? O_FP16 : O_FP32; }

bfq_status select_tile(int64_t M, int64_t N, int64_t K, int qtype, int wlayout, int sfmt,
                       bfq_tile* out) {
    if (batch_invariant()) {
        *out = invariant_tile(M, wlayout, sfmt);
        return BFQ_OK;
    }
    ensure_table();
    {
        std::lock_guard<std::mutex> lk(g_table_mu);
        auto it = g_table.entries.find(TableKey{N, K, qtype, wlayout, sfmt});
        if (it != g_table.entries.end()) {
            *out = it->second.at(nearest_bucket(it->second, M));
            out->bk = 128;
            return BFQ_OK;
        }
    }
    *out = default_tile(M, N, K, qtype, wlayout, sfmt);
    if (std::getenv("BFQ_LOG"))
        std::fprintf(stderr, "[bfq] no tuned entry for N=%lld K=%lld layout=%d scales=%d; using default tile\n",
                     (long long)N, (long long)K, wlayout, sfmt);
    return BFQ_WARN_DEFAULT_TILE;
}

// Grouped (MoE) selection: the (E, N, K, dtype, layout, scales) entry, nearest bucket to the
// token count T; batch-invariant mode as for dense tiles, keyed by the average rows per
// active expert (every grouped tile it names is compiled); else the default rule + warning.
bfq_status moe_select_tile(int64_t T, int64_t topk, int64_t E, int64_t N, int64_t K, int qtype,
                           int wlayout, int sfmt, bfq_tile* out) {
    const int64_t pairs = T * topk, active = E < pairs ? E : pairs;
    if (batch_invariant()) {
        *out = invariant_tile(active > 0 ? (pairs + active - 1) / active : 1, wlayout, sfmt);
        out->group_m = 1;
        if (out->variant == 0 && out->bm == 256) {   // grouped 256x256 is sched 1 only
            out->bm = 128; out->waves_m = 2;
        }
        return BFQ_OK;
    }
    ensure_table();
    {
        std::lock_guard<std::mutex> lk(g_table_mu);
        auto it = g_table.entries.find(TableKey{N, K, qtype, wlayout, sfmt, E});
        if (it != g_table.entries.end()) {
            *out = it->second.at(nearest_bucket(it->second, T));
            out->bk = 128;
            return BFQ_OK;
        }
    }
    *out = moe_default_tile(T, topk, E, sfmt);
    return BFQ_WARN_DEFAULT_TILE;
}

// Scale granularity from block_shape ([BENCH] §4.2 block_size; [HELION] scope section):
// {128, 128} = 1x128 token groups and 128x128 weight blocks; {1, K} = one scale per token and
// one per output channel (K <= kChannelMaxK). Sets *sfmt to S_CHANNEL for the latter.
bool scale_mode(const int32_t* bs, int64_t K, int* sfmt) {
    if (!bs) return false;
    if (bs[0] == 128 && bs[1] == 128) return true;
    if (bs[0] == 1 && bs[1] > 0 && bs[1] == K && K <= kChannelMaxK) {
        *sfmt = S_CHANNEL;
        return true;
    }
    return false;
}

bool block_shape_ok(const int32_t* bs) { return bs && bs[0] == 128 && bs[1] == 128; }

const char* kBlockShapeMsg =
    "block_shape must be {128, 128} or {1, K} (per-channel, K a multiple of 128 up to 32768)";

bool wlayout_ok(bfq_weight_layout w) { return w == BFQ_W_ROW_MAJOR || w == BFQ_W_PACKED16; }

bool sfmt_ok(bfq_scale_format f) { return f == BFQ_SCALE_FP32 || f == BFQ_SCALE_UE8M0; }

size_t workspace_for(int64_t M, int64_t N, const bfq_tile& t) {
    if (too_many_outputs(M, N)) return SIZE_MAX;   // a shape the GEMM rejects
    if (t.variant == 2) {
        if (M == 0 || t.bm <= 0 || t.bn <= 0) return 0;
        return streamk_workspace_bytes(t.bm, t.bn, streamk_grid());
    }
    return t.split_k > 1 ? (size_t)t.split_k * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// ------------------------------------------------------ allocation-free entry point ----
// The workspace of bfq_block_gemm_noalloc: a device array of this file, one copy per GPU,
// resident from the library's load until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: its device address on the current GPU comes from
// hipGetSymbolAddress (looked up once per device, on the first call that needs it) and only
// that address is ever handed to a kernel. Every call on one GPU shares the array, so calls
// that overlap on one GPU race; nothing in it needs to start at zero (split-K partials and
// stream-K slots are written before they are read).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

// A selected tile made to fit the static scratch: stream-K becomes the plain grid of the same
// tile (when that kernel is compiled), and the K split drops until its partials fit.
bfq_tile fit_scratch(bfq_tile t, int64_t M, int64_t N, int qtype, int otype, int wl, int sf) {
    if (t.variant == 2 && workspace_for(M, N, t) > kNoAllocScratchBytes) {
        bfq_tile p = t;
        p.variant = 0;
        p.split_k = 1;
        if (find_kernel(p, qtype, otype, wl, sf)) t = p;
    }
    while (t.variant != 2 && t.split_k > 1 && workspace_for(M, N, t) > kNoAllocScratchBytes)
        --t.split_k;
    return t;
}

}  // namespace

// ================================================================== C-ABI ====

extern "C" {

const char* bfq_status_string(bfq_status s) {
    switch (s) {
        case BFQ_OK: return "BFQ_OK";
        case BFQ_WARN_DEFAULT_TILE: return "BFQ_WARN_DEFAULT_TILE";
        case BFQ_ERR_NULL: return "BFQ_ERR_NULL";
        case BFQ_ERR_SHAPE: return "BFQ_ERR_SHAPE";
        case BFQ_ERR_DTYPE: return "BFQ_ERR_DTYPE";
        case BFQ_ERR_ALIGN: return "BFQ_ERR_ALIGN";
        case BFQ_ERR_WORKSPACE: return "BFQ_ERR_WORKSPACE";
        case BFQ_ERR_TILE: return "BFQ_ERR_TILE";
        case BFQ_ERR_TABLE: return "BFQ_ERR_TABLE";
        case BFQ_ERR_HIP: return "BFQ_ERR_HIP";
        case BFQ_ERR_ARG: return "BFQ_ERR_ARG";
    }
    return "BFQ_UNKNOWN_STATUS";
}

const char* bfq_last_error(void) { return g_last_error.c_str(); }

void bfq_set_batch_invariant(int32_t enable) { g_batch_invariant = enable ? 1 : 0; }

int32_t bfq_get_batch_invariant(void) { return batch_invariant() ? 1 : 0; }

bfq_status bfq_quant_tokens(const void* x_bf16, int64_t M, int64_t K, int32_t group_size,
                            bfq_dtype q_dtype, void* q, float* scales, bfq_scale_layout layout,
                            int64_t scale_ld, float eps, bfq_scale_format scale_fmt,
                            void* stream) {
    if (M != 0 && (!x_bf16 || !q || !scales))
        return fail(BFQ_ERR_NULL, "x, q and scales must be non-NULL");
    if (q_dtype != BFQ_E4M3FN && q_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "q_dtype must be BFQ_E4M3FN or BFQ_INT8");
    if (M < 0 || K <= 0 || K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "need M >= 0 and K a positive multiple of 128");
    const bool per_token = group_size == K && K != 128;
    if (group_size != 128 && !(per_token && K <= kChannelMaxK))
        return fail(BFQ_ERR_SHAPE, "group_size must be 128 or K (per token, K <= 32768)");
    if (M > 0x7FFFFFFF) return fail(BFQ_ERR_SHAPE, "M exceeds 2^31 - 1");
    if (!aligned(x_bf16, 16) || !aligned(q, 16) || !aligned(scales, 4))
        return fail(BFQ_ERR_ALIGN, "x and q must be 16-byte aligned, scales 4-byte aligned");
    if (!(eps > 0.0f) || eps > 3.0e38f) return fail(BFQ_ERR_ARG, "eps must be positive and finite");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    const int64_t G = K / group_size;
    int64_t sm, sg;
    const bool packed = layout == BFQ_SCALES_PACKED_UE8M0;
    if (layout == BFQ_SCALES_ROW_MAJOR) {
        if (scale_ld < G) return fail(BFQ_ERR_SHAPE, "row-major scale_ld must be >= K/group_size");
        sm = scale_ld; sg = 1;
    } else if (layout == BFQ_SCALES_COL_MAJOR) {
        if (scale_ld < M) return fail(BFQ_ERR_SHAPE, "column-major scale_ld must be >= M");
        sm = 1; sg = scale_ld;
    } else if (packed) {
        if (scale_fmt != BFQ_SCALE_UE8M0 || per_token)
            return fail(BFQ_ERR_ARG, "packed scale words need UE8M0 scales of 1x128 groups");
        if (scale_ld < (M + 3) / 4 * 4)
            return fail(BFQ_ERR_SHAPE, "packed scale_ld must be >= M rounded up to a multiple of 4");
        sm = 1; sg = scale_ld;
    } else {
        return fail(BFQ_ERR_ARG, "unknown scale layout");
    }
    if (M == 0) return BFQ_OK;
    hipError_t e = per_token
                       ? launch_quant_rows(x_bf16, 0, q, scales, M, K, qtype_of(q_dtype), sm, eps,
                                           (int)scale_fmt, (hipStream_t)stream)
                       : launch_quant_tokens(x_bf16, q, scales, M, K, qtype_of(q_dtype), sm, sg,
                                             eps, (int)scale_fmt, packed ? 1 : 0,
                                             (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

bfq_status bfq_quant_weight_blocks(const float* w, int64_t N, int64_t K,
                                   const int32_t block_shape[2], bfq_dtype q_dtype, void* q,
                                   float* scales, float eps, bfq_scale_format scale_fmt,
                                   void* stream) {
    if (!w || !q || !scales || !block_shape)
        return fail(BFQ_ERR_NULL, "w, q, scales and block_shape must be non-NULL");
    if (q_dtype != BFQ_E4M3FN && q_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "q_dtype must be BFQ_E4M3FN or BFQ_INT8");
    int wsf = S_FP32;
    if (!scale_mode(block_shape, K, &wsf)) return fail(BFQ_ERR_SHAPE, kBlockShapeMsg);
    if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "N and K must be non-negative multiples of 128");
    if (N / 128 > 65535 || K / 128 > 0x7FFFFFFF) return fail(BFQ_ERR_SHAPE, "N or K too large");
    if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scales, 4))
        return fail(BFQ_ERR_ALIGN, "w and q must be 16-byte aligned, scales 4-byte aligned");
    if (!(eps > 0.0f) || eps > 3.0e38f) return fail(BFQ_ERR_ARG, "eps must be positive and finite");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    if (N == 0 || K == 0) return BFQ_OK;
    hipError_t e = wsf == S_CHANNEL
                       ? launch_quant_rows(w, 1, q, scales, N, K, qtype_of(q_dtype), 1, eps,
                                           (int)scale_fmt, (hipStream_t)stream)
                       : launch_quant_weight_blocks(w, q, scales, N, K, qtype_of(q_dtype), eps,
                                                    (int)scale_fmt, (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

bfq_status bfq_pack_weights(const void* w_q, int64_t N, int64_t K, bfq_dtype q_dtype,
                            void* w_packed, void* stream) {
    if (!w_q || !w_packed) return fail(BFQ_ERR_NULL, "w_q and w_packed must be non-NULL");
    if (q_dtype != BFQ_E4M3FN && q_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "q_dtype must be BFQ_E4M3FN or BFQ_INT8");
    if (N < 0 || K < 0 || N % 128 != 0 || K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "N and K must be non-negative multiples of 128");
    if (N > 0x7FFFFFFF || K > 0x7FFFFFFF || N * K / 4096 > 0x7FFFFFFF)
        return fail(BFQ_ERR_SHAPE, "N * K too large (one 256-thread block per 4 KiB)");
    if (!aligned(w_q, 16) || !aligned(w_packed, 16))
        return fail(BFQ_ERR_ALIGN, "w_q and w_packed must be 16-byte aligned");
    const uintptr_t a = (uintptr_t)w_q, b = (uintptr_t)w_packed, n = (uintptr_t)(N * K);
    if (n > 0 && a < b + n && b < a + n)
        return fail(BFQ_ERR_ARG, "w_q and w_packed must not overlap");
    if (N == 0 || K == 0) return BFQ_OK;
    hipError_t e = launch_pack_weights(w_q, w_packed, N, K, (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

bfq_status bfq_select_tile(int64_t M, int64_t N, int64_t K, const int32_t block_shape[2],
                           bfq_dtype in_dtype, bfq_dtype out_dtype, bfq_weight_layout w_layout,
                           bfq_scale_format scale_fmt, bfq_tile* tile_out) {
    if (!tile_out || !block_shape) return fail(BFQ_ERR_NULL, "tile_out and block_shape must be non-NULL");
    int sf = (int)scale_fmt;
    if (!scale_mode(block_shape, K, &sf)) return fail(BFQ_ERR_SHAPE, kBlockShapeMsg);
    if (in_dtype != BFQ_E4M3FN && in_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "in_dtype must be BFQ_E4M3FN or BFQ_INT8");
    if (out_dtype != BFQ_BF16 && out_dtype != BFQ_FP16 && out_dtype != BFQ_FP32)
        return fail(BFQ_ERR_DTYPE, "out_dtype must be BF16, FP16 or FP32");
    if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "need M >= 0 and N, K positive multiples of 128");
    if (!wlayout_ok(w_layout)) return fail(BFQ_ERR_ARG, "unknown weight layout");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    return select_tile(M, N, K, qtype_of(in_dtype), (int)w_layout, sf, tile_out);
}

size_t bfq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const bfq_tile* tile) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    bfq_tile t;
    if (tile) t = *tile;
    else select_tile(M, N, K, Q_FP8, W_ROW, S_FP32, &t);
    return workspace_for(M, N, t);
}

}  // extern "C"

namespace {

// The block GEMM behind bfq_block_gemm and bfq_block_gemm_noalloc. noalloc: the workspace is
// the library's static scratch (kNoAllocScratchBytes); a selected (tile == NULL) tile whose
// workspace would not fit it is reduced to one that does, an explicit one is rejected.
bfq_status block_gemm_impl(const void* a_q, const float* a_scales, bfq_scale_layout a_layout,
                           int64_t a_scale_ld, const void* w_q, const float* w_scales,
                           bfq_weight_layout w_layout, bfq_scale_format scale_fmt, void* out,
                           int64_t M, int64_t N, int64_t K, const int32_t block_shape[2],
                           bfq_dtype in_dtype, bfq_dtype out_dtype, const bfq_tile* tile,
                           void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
    if (!w_q || !w_scales || !block_shape || (M != 0 && (!a_q || !a_scales || !out)))
        return fail(BFQ_ERR_NULL, "a_q, a_scales, w_q, w_scales, out and block_shape must be non-NULL");
    int sf = (int)scale_fmt;
    if (!scale_mode(block_shape, K, &sf)) return fail(BFQ_ERR_SHAPE, kBlockShapeMsg);
    const bool channel = sf == S_CHANNEL;
    if (in_dtype != BFQ_E4M3FN && in_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "in_dtype must be BFQ_E4M3FN or BFQ_INT8");
    if (out_dtype != BFQ_BF16 && out_dtype != BFQ_FP16 && out_dtype != BFQ_FP32)
        return fail(BFQ_ERR_DTYPE, "out_dtype must be BF16, FP16 or FP32");
    if (!wlayout_ok(w_layout)) return fail(BFQ_ERR_ARG, "unknown weight layout");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "need M >= 0 and N, K positive multiples of 128");
    if (M > 0x7FFFFFFF || N > 0x7FFFFFFF || K > (1 << 23))
        return fail(BFQ_ERR_SHAPE, "M and N must be below 2^31 and K at most 2^23");
    if (too_many_outputs(M, N)) return fail(BFQ_ERR_SHAPE, "M * N must be below 2^40");
    if (a_scale_ld > (1 << 23)) return fail(BFQ_ERR_SHAPE, "a_scale_ld must be at most 2^23");
    if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(out, 16) || !aligned(a_scales, 4) ||
        !aligned(w_scales, 4) || !aligned(workspace, 16))
        return fail(BFQ_ERR_ALIGN, "codes, out and workspace must be 16-byte aligned, scales 4-byte");
    const int64_t KB = K / 128;
    const int64_t G = channel ? 1 : KB;   // activation scales per token
    int64_t ssm, ssk;
    if (a_layout == BFQ_SCALES_ROW_MAJOR) {
        if (a_scale_ld < G)
            return fail(BFQ_ERR_SHAPE, "row-major a_scale_ld must be >= K/128 (per token: >= 1)");
        ssm = a_scale_ld; ssk = channel ? 0 : 1;
    } else if (a_layout == BFQ_SCALES_COL_MAJOR) {
        if (a_scale_ld < M) return fail(BFQ_ERR_SHAPE, "column-major a_scale_ld must be >= M");
        ssm = 1; ssk = channel ? 0 : a_scale_ld;
    } else if (a_layout == BFQ_SCALES_PACKED_UE8M0) {
        if (channel || scale_fmt != BFQ_SCALE_UE8M0)
            return fail(BFQ_ERR_ARG, "packed scale words need block scales in the UE8M0 format");
        if (in_dtype != BFQ_E4M3FN)
            return fail(BFQ_ERR_DTYPE, "packed scale words are read by the e4m3fn GEMM only");
        if (a_scale_ld < M) return fail(BFQ_ERR_SHAPE, "packed a_scale_ld must be >= M");
        ssm = 1; ssk = a_scale_ld;      // words between word rows (4 K blocks each)
    } else {
        return fail(BFQ_ERR_ARG, "unknown scale layout");
    }
    // the kernels address the activation scales of one tile (at most 256 tokens, all K
    // blocks) with 32-bit byte offsets
    const int64_t k_rows = a_layout == BFQ_SCALES_PACKED_UE8M0 ? (KB - 1) / 4 : KB - 1;
    if ((255 * ssm + k_rows * ssk + 1) * 4 >= (int64_t(1) << 32))
        return fail(BFQ_ERR_SHAPE, "activation scales of 256 tokens must span less than 4 GiB");
    const int qtype = qtype_of(in_dtype), otype = otype_of(out_dtype), wl = (int)w_layout;
    bfq_status status = BFQ_OK;
    bfq_tile t;
    if (tile) {
        t = *tile;
    } else {
        status = select_tile(M, N, K, qtype, wl, sf, &t);
    }
    // a packed-word tile is selected like a UE8M0 one, then served by a kernel that reads words
    const int ksf = a_layout == BFQ_SCALES_PACKED_UE8M0 ? S_PACKED : sf;
    if (noalloc && !tile) t = fit_scratch(t, M, N, qtype, otype, wl, ksf);
    const KernelEntry* ke = find_kernel(t, qtype, otype, wl, ksf);
    if (!ke)
        return fail(BFQ_ERR_TILE, "tile does not name a compiled kernel for this dtype pair, weight "
                                  "layout and scale format / granularity");
    if (t.split_k < 1 || t.split_k > 256 || t.split_k > KB)
        return fail(BFQ_ERR_TILE, "split_k must be in [1, min(256, K/128)]");
    if (t.variant == 2 && t.split_k != 1)
        return fail(BFQ_ERR_TILE, "the stream-K schedule (variant 2) takes split_k = 1");
    if (t.variant != 1 && (t.group_m < 1 || t.raster < 0 || t.raster > 1))
        return fail(BFQ_ERR_TILE, "group_m must be >= 1 and raster 0 or 1");
    const size_t need = workspace_for(M, N, t);
    if (noalloc && need > kNoAllocScratchBytes)
        return fail(BFQ_ERR_WORKSPACE, "the tile needs " + std::to_string(need) +
                                           " bytes of workspace; the allocation-free entry point "
                                           "holds " + std::to_string(kNoAllocScratchBytes));
    if (!noalloc && need > 0 && (!workspace || workspace_bytes < need))
        return fail(BFQ_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
    // grid-size limits of the launchers
    if (t.variant != 1) {
        int64_t tiles = ceil_div(M, t.bm) * ceil_div(N, t.bn);
        if (tiles > 0x7FFFFFFF) return fail(BFQ_ERR_SHAPE, "too many output tiles");
    } else if (ceil_div(M, t.bm) > 65535) {
        return fail(BFQ_ERR_SHAPE, "M too large for the swap-AB kernel; use a standard tile");
    }
    if (M == 0) return status;
    if (noalloc && need > 0) {
        hipError_t e = scratch_on_current_device(&workspace);
        if (e != hipSuccess) return fail(BFQ_ERR_HIP, std::string("scratch lookup: ") + hipGetErrorString(e));
    }

    GemmArgs ga;
    ga.a = a_q;
    ga.sa = a_scales;
    ga.sa_stride_m = ssm;
    ga.sa_stride_k = ssk;
    ga.sa_packed = a_layout == BFQ_SCALES_PACKED_UE8M0 ? 1 : 0;
    ga.w = w_q;
    ga.sw = w_scales;
    ga.out = out;
    ga.partials = static_cast<float*>(workspace);
    ga.M = M;
    ga.N = N;
    ga.K = K;
    ga.split = t.split_k;
    ga.group_m = t.group_m;
    ga.raster = t.raster;
    ga.dp_tiles = 0;
    ga.sk_slots = nullptr;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = ke->launch(ga, s);
    if (e == hipSuccess && t.split_k > 1)
        e = launch_splitk_reduce(ga.partials, out, M, N, t.split_k, otype, s);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    if (std::getenv("BFQ_TRACE"))
        std::fprintf(stderr, "[bfq] gemm M=%lld N=%lld K=%lld layout=%d scales=%d variant=%d bm=%d bn=%d split=%d\n",
                     (long long)M, (long long)N, (long long)K, wl, sf, t.variant, t.bm, t.bn, t.split_k);
    return status;
}

}  // namespace

extern "C" {

bfq_status bfq_block_gemm(const void* a_q, const float* a_scales, bfq_scale_layout a_layout,
                          int64_t a_scale_ld, const void* w_q, const float* w_scales,
                          bfq_weight_layout w_layout, bfq_scale_format scale_fmt, void* out,
                          int64_t M, int64_t N, int64_t K, const int32_t block_shape[2],
                          bfq_dtype in_dtype, bfq_dtype out_dtype, const bfq_tile* tile,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return block_gemm_impl(a_q, a_scales, a_layout, a_scale_ld, w_q, w_scales, w_layout,
                           scale_fmt, out, M, N, K, block_shape, in_dtype, out_dtype, tile,
                           workspace, workspace_bytes, stream, false);
}

bfq_status bfq_block_gemm_noalloc(const void* a_q, const float* a_scales,
                                  bfq_scale_layout a_layout, int64_t a_scale_ld, const void* w_q,
                                  const float* w_scales, bfq_weight_layout w_layout,
                                  bfq_scale_format scale_fmt, void* out, int64_t M, int64_t N,
                                  int64_t K, const int32_t block_shape[2], bfq_dtype in_dtype,
                                  bfq_dtype out_dtype, const bfq_tile* tile, void* stream) {
    return block_gemm_impl(a_q, a_scales, a_layout, a_scale_ld, w_q, w_scales, w_layout,
                           scale_fmt, out, M, N, K, block_shape, in_dtype, out_dtype, tile,
                           nullptr, 0, stream, true);
}

size_t bfq_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

bfq_status bfq_load_tile_table(const char* json_path) {
    std::lock_guard<std::mutex> lk(g_table_mu);
    if (!json_path) return load_table_locked(default_table_path(), false);
    return load_table_locked(json_path, true);
}

// block_shape {1, k} (any k > 0) selects the per-token x per-channel kernels here
static int candidate_sfmt(const int32_t* bs, bfq_scale_format f) {
    if (!bs) return -1;
    if (bs[0] == 128 && bs[1] == 128) return (int)f;
    if (bs[0] == 1 && bs[1] > 0) return S_CHANNEL;
    return -1;
}

int32_t bfq_num_tile_candidates(const int32_t block_shape[2], bfq_dtype in_dtype,
                                bfq_weight_layout w_layout, bfq_scale_format scale_fmt) {
    if (in_dtype != BFQ_E4M3FN && in_dtype != BFQ_INT8) return 0;
    if (!wlayout_ok(w_layout) || !sfmt_ok(scale_fmt)) return 0;
    const int sf = candidate_sfmt(block_shape, scale_fmt);
    if (sf < 0) return 0;
    const int q = qtype_of(in_dtype), wl = (int)w_layout;
    int ns[3] = {0, 0, 0}, count = 0;
    const KernelEntry* lists[3] = {std_kernels(&ns[0]), swapab_kernels(&ns[1]), streamk_kernels(&ns[2])};
    for (int l = 0; l < 3; ++l)
        for (int i = 0; i < ns[l]; ++i)
            count += (lists[l][i].qtype == q && lists[l][i].otype == O_BF16 && lists[l][i].wlayout == wl &&
                      serves(lists[l][i], sf));
    return count;
}

bfq_status bfq_get_tile_candidate(const int32_t block_shape[2], bfq_dtype in_dtype,
                                  bfq_weight_layout w_layout, bfq_scale_format scale_fmt,
                                  int32_t index, bfq_tile* tile_out) {
    if (!tile_out || !block_shape) return fail(BFQ_ERR_NULL, "tile_out and block_shape must be non-NULL");
    const int sf = candidate_sfmt(block_shape, scale_fmt);
    if (sf < 0) return fail(BFQ_ERR_SHAPE, "block_shape must be {128, 128} or {1, k}");
    if (in_dtype != BFQ_E4M3FN && in_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "in_dtype must be BFQ_E4M3FN or BFQ_INT8");
    if (!wlayout_ok(w_layout)) return fail(BFQ_ERR_ARG, "unknown weight layout");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    const int q = qtype_of(in_dtype), wl = (int)w_layout;
    int ns[3] = {0, 0, 0}, count = 0;
    const KernelEntry* lists[3] = {std_kernels(&ns[0]), swapab_kernels(&ns[1]), streamk_kernels(&ns[2])};
    for (int l = 0; l < 3; ++l)
        for (int i = 0; i < ns[l]; ++i) {
            if (lists[l][i].qtype != q || lists[l][i].otype != O_BF16 || lists[l][i].wlayout != wl ||
                !serves(lists[l][i], sf))
                continue;
            if (count == index) { *tile_out = lists[l][i].tile; return BFQ_OK; }
            ++count;
        }
    return fail(BFQ_ERR_ARG, "candidate index out of range");
}

// ----------------------------------------------------------- MoE grouped GEMM ----

size_t bfq_moe_align_workspace_bytes(int64_t T, int32_t topk, int32_t E) {
    if (T <= 0 || topk <= 0 || E <= 0) return 0;
    return moe_align_workspace_bytes(T * topk, E);
}

bfq_status bfq_moe_align(const int32_t* topk_ids, int64_t T, int32_t topk, int32_t E,
                         int32_t* expert_offsets, int32_t* sorted_pairs, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!expert_offsets || (T > 0 && (!topk_ids || !sorted_pairs)))
        return fail(BFQ_ERR_NULL, "topk_ids, expert_offsets and sorted_pairs must be non-NULL");
    if (T < 0 || topk < 1 || E < 1 || E > kMoeMaxExperts)
        return fail(BFQ_ERR_SHAPE, "need T >= 0, topk >= 1 and 1 <= E <= 1023");
    if (T * (int64_t)topk > 0x7FFFFFFF) return fail(BFQ_ERR_SHAPE, "T * topk must be below 2^31");
    if (!aligned(topk_ids, 4) || !aligned(expert_offsets, 4) || !aligned(sorted_pairs, 4) ||
        !aligned(workspace, 4))
        return fail(BFQ_ERR_ALIGN, "int32 buffers must be 4-byte aligned");
    const size_t need = moe_align_workspace_bytes(T * topk, E);
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(BFQ_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
    hipError_t e = launch_moe_align(topk_ids, T * topk, E, expert_offsets, sorted_pairs,
                                    static_cast<int32_t*>(workspace), (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

bfq_status bfq_moe_select_tile(int64_t T, int32_t topk, int32_t E, int64_t N, int64_t K,
                               const int32_t block_shape[2], bfq_dtype in_dtype,
                               bfq_dtype out_dtype, bfq_weight_layout w_layout,
                               bfq_scale_format scale_fmt, bfq_tile* tile_out) {
    if (!tile_out || !block_shape) return fail(BFQ_ERR_NULL, "tile_out and block_shape must be non-NULL");
    if (!block_shape_ok(block_shape)) return fail(BFQ_ERR_SHAPE, "grouped GEMM: block_shape must be {128, 128}");
    if (in_dtype != BFQ_E4M3FN) return fail(BFQ_ERR_DTYPE, "grouped GEMM: in_dtype must be BFQ_E4M3FN");
    if (out_dtype != BFQ_BF16 && out_dtype != BFQ_FP16 && out_dtype != BFQ_FP32)
        return fail(BFQ_ERR_DTYPE, "out_dtype must be BF16, FP16 or FP32");
    if (T < 0 || topk < 1 || E < 1 || E > kMoeMaxExperts || N <= 0 || K <= 0 || N % 128 != 0 ||
        K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "need T >= 0, topk >= 1, 1 <= E <= 1023, N and K positive multiples of 128");
    if (!wlayout_ok(w_layout)) return fail(BFQ_ERR_ARG, "unknown weight layout");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    return moe_select_tile(T, topk, E, N, K, Q_FP8, (int)w_layout, (int)scale_fmt, tile_out);
}

size_t bfq_moe_gemm_workspace_bytes(int64_t T, int32_t topk, int64_t N, const bfq_tile* tile) {
    if (!tile || T <= 0 || topk <= 0 || N <= 0 || tile->split_k <= 1) return 0;
    if (too_many_outputs(T, topk) || too_many_outputs(T * topk, N)) return SIZE_MAX;
    return (size_t)tile->split_k * (size_t)(T * topk) * (size_t)N * sizeof(float);
}

bfq_status bfq_moe_block_gemm(const void* a_q, const float* a_scales, bfq_scale_layout a_layout,
                              int64_t a_scale_ld, const int32_t* sorted_pairs,
                              const int32_t* expert_offsets, int32_t topk, const void* w_q,
                              const float* w_scales, bfq_weight_layout w_layout,
                              bfq_scale_format scale_fmt, void* out, int64_t T, int64_t N,
                              int64_t K, int32_t E, const int32_t block_shape[2],
                              bfq_dtype in_dtype, bfq_dtype out_dtype, const bfq_tile* tile,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!w_q || !w_scales || !block_shape || !expert_offsets ||
        (T != 0 && (!a_q || !a_scales || !out || !sorted_pairs)))
        return fail(BFQ_ERR_NULL, "a_q, a_scales, sorted_pairs, expert_offsets, w_q, w_scales, out "
                                  "and block_shape must be non-NULL");
    if (!block_shape_ok(block_shape)) return fail(BFQ_ERR_SHAPE, "grouped GEMM: block_shape must be {128, 128}");
    if (in_dtype != BFQ_E4M3FN) return fail(BFQ_ERR_DTYPE, "grouped GEMM: in_dtype must be BFQ_E4M3FN");
    if (out_dtype != BFQ_BF16 && out_dtype != BFQ_FP16 && out_dtype != BFQ_FP32)
        return fail(BFQ_ERR_DTYPE, "out_dtype must be BF16, FP16 or FP32");
    if (!wlayout_ok(w_layout)) return fail(BFQ_ERR_ARG, "unknown weight layout");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    if (T < 0 || topk < 1 || E < 1 || E > kMoeMaxExperts || N <= 0 || K <= 0 || N % 128 != 0 ||
        K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "need T >= 0, topk >= 1, 1 <= E <= 1023, N and K positive multiples of 128");
    const int64_t P = T * topk;
    // the kernels gather token rows through one 32-bit offset over all of a_q, and address
    // up to 256 weight rows of an expert (and a K block's offset) in 32 bits, as the dense
    // kernels do
    if (T * K >= (int64_t(1) << 31) || P > 0x7FFFFFFF || N > 0x7FFFFFFF)
        return fail(BFQ_ERR_SHAPE, "T * K must be below 2^31 bytes");
    if (too_many_outputs(P, N)) return fail(BFQ_ERR_SHAPE, "T * topk * N must be below 2^40");
    if (K > (1 << 23)) return fail(BFQ_ERR_SHAPE, "K must be at most 2^23");
    if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(out, 16) || !aligned(a_scales, 4) ||
        !aligned(w_scales, 4) || !aligned(workspace, 16) || !aligned(sorted_pairs, 4) ||
        !aligned(expert_offsets, 4))
        return fail(BFQ_ERR_ALIGN, "codes, out and workspace must be 16-byte aligned, scales and int32 arrays 4-byte");
    const int64_t KB = K / 128;
    int64_t ssm, ssk;
    const bool packed = a_layout == BFQ_SCALES_PACKED_UE8M0;
    if (a_layout == BFQ_SCALES_ROW_MAJOR) {
        if (a_scale_ld < KB) return fail(BFQ_ERR_SHAPE, "row-major a_scale_ld must be >= K/128");
        ssm = a_scale_ld; ssk = 1;
    } else if (a_layout == BFQ_SCALES_COL_MAJOR) {
        if (a_scale_ld < T) return fail(BFQ_ERR_SHAPE, "column-major a_scale_ld must be >= T");
        ssm = 1; ssk = a_scale_ld;
    } else if (packed) {
        if (scale_fmt != BFQ_SCALE_UE8M0)
            return fail(BFQ_ERR_ARG, "packed scale words need scales in the UE8M0 format");
        if (a_scale_ld < T) return fail(BFQ_ERR_SHAPE, "packed a_scale_ld must be >= T");
        ssm = 1; ssk = a_scale_ld;
    } else {
        return fail(BFQ_ERR_ARG, "unknown scale layout");
    }
    const int64_t k_rows = packed ? (KB - 1) / 4 : KB - 1;
    if (T > 0 && ((T - 1) * ssm + k_rows * ssk + 1) * 4 >= (int64_t(1) << 31))
        return fail(BFQ_ERR_SHAPE, "the activation scales must span less than 2 GiB");
    const int wl = (int)w_layout, sf = (int)scale_fmt, otype = otype_of(out_dtype);
    bfq_status status = BFQ_OK;
    bfq_tile t;
    if (tile) t = *tile;
    else status = moe_select_tile(T, topk, E, N, K, Q_FP8, wl, sf, &t);
    const KernelEntry* ke = find_kernel(t, Q_FP8, otype, wl, packed ? S_PACKED : sf, 1);
    if (!ke)
        return fail(BFQ_ERR_TILE, "tile does not name a compiled grouped kernel for this weight "
                                  "layout and scale format");
    if (t.split_k < 1 || t.split_k > 256 || t.split_k > KB)
        return fail(BFQ_ERR_TILE, "split_k must be in [1, min(256, K/128)]");
    if (moe_max_tiles(P, E, t.bm) > 65535)
        return fail(BFQ_ERR_SHAPE, "too many row tiles for one grouped launch");
    const size_t need = t.split_k > 1 ? (size_t)t.split_k * (size_t)P * (size_t)N * sizeof(float) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need))
        return fail(BFQ_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
    if (P == 0) return status;

    GemmArgs ga{};
    ga.a = a_q;
    ga.sa = a_scales;
    ga.sa_stride_m = ssm;
    ga.sa_stride_k = ssk;
    ga.sa_packed = packed ? 1 : 0;
    ga.w = w_q;
    ga.sw = w_scales;
    ga.out = out;
    ga.partials = static_cast<float*>(workspace);
    ga.M = P;
    ga.N = N;
    ga.K = K;
    ga.split = t.split_k;
    ga.group_m = 1;
    ga.raster = 0;
    ga.moe_rows = sorted_pairs;
    ga.moe_offsets = expert_offsets;
    ga.moe_tokens = T;
    ga.moe_topk = topk;
    ga.moe_experts = E;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = ke->launch(ga, s);
    if (e == hipSuccess && t.split_k > 1)
        e = launch_splitk_reduce(ga.partials, out, P, N, t.split_k, otype, s);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return status;
}

int32_t bfq_moe_num_tile_candidates(bfq_weight_layout w_layout, bfq_scale_format scale_fmt) {
    if (!wlayout_ok(w_layout) || !sfmt_ok(scale_fmt)) return 0;
    int ns[2] = {0, 0}, count = 0;
    const KernelEntry* lists[2] = {moe_std_kernels(&ns[0]), moe_swapab_kernels(&ns[1])};
    for (int l = 0; l < 2; ++l)
        for (int i = 0; i < ns[l]; ++i)
            count += (lists[l][i].otype == O_BF16 && lists[l][i].wlayout == (int)w_layout &&
                      serves(lists[l][i], (int)scale_fmt));
    return count;
}

bfq_status bfq_moe_get_tile_candidate(bfq_weight_layout w_layout, bfq_scale_format scale_fmt,
                                      int32_t index, bfq_tile* tile_out) {
    if (!tile_out) return fail(BFQ_ERR_NULL, "tile_out must be non-NULL");
    if (!wlayout_ok(w_layout)) return fail(BFQ_ERR_ARG, "unknown weight layout");
    if (!sfmt_ok(scale_fmt)) return fail(BFQ_ERR_ARG, "unknown scale format");
    int ns[2] = {0, 0}, count = 0;
    const KernelEntry* lists[2] = {moe_std_kernels(&ns[0]), moe_swapab_kernels(&ns[1])};
    for (int l = 0; l < 2; ++l)
        for (int i = 0; i < ns[l]; ++i) {
            if (lists[l][i].otype != O_BF16 || lists[l][i].wlayout != (int)w_layout ||
                !serves(lists[l][i], (int)scale_fmt))
                continue;
            if (count == index) { *tile_out = lists[l][i].tile; return BFQ_OK; }
            ++count;
        }
    return fail(BFQ_ERR_ARG, "candidate index out of range");
}

bfq_status bfq_debug_block_partials_i32(const void* a_q, const void* w_q, int32_t* partials,
                                        int64_t M, int64_t N, int64_t K, void* stream) {
    if (!w_q || (M != 0 && (!a_q || !partials)))
        return fail(BFQ_ERR_NULL, "a_q, w_q and partials must be non-NULL");
    if (M < 0 || N <= 0 || K <= 0 || N % 128 != 0 || K % 128 != 0)
        return fail(BFQ_ERR_SHAPE, "need M >= 0 and N, K positive multiples of 128");
    if ((M + 15) / 16 > 65535 || K / 128 > 65535) return fail(BFQ_ERR_SHAPE, "shape too large");
    if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(partials, 16))
        return fail(BFQ_ERR_ALIGN, "buffers must be 16-byte aligned");
    if (M == 0) return BFQ_OK;
    hipError_t e = launch_block_partials_i32(a_q, w_q, partials, M, N, K, (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

bfq_status bfq_probe_mfma_peak(int64_t blocks, int64_t iters, float* out, void* stream) {
    if (!out) return fail(BFQ_ERR_NULL, "out must be non-NULL");
    if (blocks < 1 || blocks >= (int64_t(1) << 31) || iters < 1 || iters >= (int64_t(1) << 40))
        return fail(BFQ_ERR_SHAPE, "blocks must be in [1, 2^31) and iters in [1, 2^40)");
    if (!aligned(out, 4)) return fail(BFQ_ERR_ALIGN, "out must be 4-byte aligned");
    hipError_t e = launch_mfma_peak(blocks, iters, out, (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

double bfq_probe_mfma_flops(int64_t blocks, int64_t iters) {
    const double waves = (double)blocks * (mfma_peak_threads_per_block() / 64);
    return waves * (double)iters * mfma_peak_mfmas_per_wave_iter() * (2.0 * 16 * 16 * 128);
}

bfq_status bfq_debug_encode(const float* x, int64_t n, bfq_dtype q_dtype, void* codes,
                            void* stream) {
    if (!x || !codes) return fail(BFQ_ERR_NULL, "x and codes must be non-NULL");
    if (q_dtype != BFQ_E4M3FN && q_dtype != BFQ_INT8)
        return fail(BFQ_ERR_DTYPE, "q_dtype must be BFQ_E4M3FN or BFQ_INT8");
    if (n < 0 || (n + 1023) / 1024 > 0x7FFFFFFF) return fail(BFQ_ERR_SHAPE, "bad element count");
    if (!aligned(x, 16) || !aligned(codes, 4)) return fail(BFQ_ERR_ALIGN, "x 16-byte, codes 4-byte aligned");
    if (n == 0) return BFQ_OK;
    hipError_t e = launch_debug_encode(x, n, qtype_of(q_dtype), codes, (hipStream_t)stream);
    if (e != hipSuccess) return fail(BFQ_ERR_HIP, hipGetErrorString(e));
    return BFQ_OK;
}

}  // extern "C"
