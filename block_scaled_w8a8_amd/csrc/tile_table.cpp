// JSON reader and nearest-M rule for the tile table (see tile_table.h for the page cited).
//
// File schema (one file holds every shape; the per-entry keys are those of the page's file
// names — N, K, dtype, block_shape — and "configs" is the page's per-file M -> launch map):
// {
//   "device": "gfx950",
//   "entries": [
//     { "N": 24576, "K": 7168, "dtype": "fp8_w8a8", "block_shape": [128, 128],
//       "w_layout": "packed16",            (optional; "row_major" when absent)
//       "scales": "ue8m0",                 (optional; "fp32" when absent; not with [1, K])
//       "E": 256,                          (optional; expert count of a grouped MoE entry,
//                                           whose M buckets are token counts; 0 when absent)
//       "configs": { "1": {"variant": 1, "bm": 16, "bn": 128, "split_k": 2, "waves_m": 1,
//                          "waves_n": 4, "stages": 4, "group_m": 1}, ... } } ] }
#include "tile_table.h"

#include <cctype>
#include <cstdlib>

namespace bfq {
namespace {

struct JVal {
    enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
    double num = 0;
    bool b = false;
    std::string str;
    std::vector<JVal> arr;
    std::vector<std::pair<std::string, JVal>> obj;
    const JVal* get(const std::string& k) const {
        for (auto& kv : obj)
            if (kv.first == k) return &kv.second;
        return nullptr;
    }
};

struct Parser {
    const std::string& s;
    size_t i = 0;
    std::string err;
    explicit Parser(const std::string& t) : s(t) {}

    void ws() { while (i < s.size() && std::isspace((unsigned char)s[i])) ++i; }
    bool fail(const char* what) {
        if (err.empty()) err = std::string(what) + " at offset " + std::to_string(i);
        return false;
    }
    bool lit(const char* w) {
        size_t n = 0;
        while (w[n]) ++n;
        if (s.compare(i, n, w) != 0) return fail("bad literal");
        i += n;
        return true;
    }
    bool string(std::string& out) {
        if (i >= s.size() || s[i] != '"') return fail("expected string");
        ++i;
        while (i < s.size() && s[i] != '"') {
            if (s[i] == '\\') {
                if (i + 1 >= s.size()) return fail("bad escape");
                out.push_back(s[i + 1]);
                i += 2;
            } else {
                out.push_back(s[i++]);
            }
        }
        if (i >= s.size()) return fail("unterminated string");
        ++i;
        return true;
    }
    bool value(JVal& v, int depth) {
        if (depth > 32) return fail("nesting too deep");
        ws();
        if (i >= s.size()) return fail("unexpected end");
        char c = s[i];
        if (c == '{') {
            v.kind = JVal::OBJ;
            ++i;
            ws();
            if (i < s.size() && s[i] == '}') { ++i; return true; }
            for (;;) {
                ws();
                std::string k;
                if (!string(k)) return false;
                ws();
                if (i >= s.size() || s[i] != ':') return fail("expected ':'");
                ++i;
                JVal sub;
                if (!value(sub, depth + 1)) return false;
                v.obj.emplace_back(std::move(k), std::move(sub));
                ws();
                if (i < s.size() && s[i] == ',') { ++i; continue; }
                if (i < s.size() && s[i] == '}') { ++i; return true; }
                return fail("expected ',' or '}'");
            }
        }
        if (c == '[') {
            v.kind = JVal::ARR;
            ++i;
            ws();
            if (i < s.size() && s[i] == ']') { ++i; return true; }
            for (;;) {
                JVal sub;
                if (!value(sub, depth + 1)) return false;
                v.arr.push_back(std::move(sub));
                ws();
                if (i < s.size() && s[i] == ',') { ++i; continue; }
                if (i < s.size() && s[i] == ']') { ++i; return true; }
                return fail("expected ',' or ']'");
            }
        }
        if (c == '"') { v.kind = JVal::STR; return string(v.str); }
        if (c == 't') { v.kind = JVal::BOOL; v.b = true; return lit("true"); }
        if (c == 'f') { v.kind = JVal::BOOL; v.b = false; return lit("false"); }
        if (c == 'n') { v.kind = JVal::NUL; return lit("null"); }
        if (c == '-' || std::isdigit((unsigned char)c)) {
            const char* b = s.c_str() + i;
            char* e = nullptr;
            v.num = std::strtod(b, &e);
            if (e == b) return fail("bad number");
            v.kind = JVal::NUM;
            i += (size_t)(e - b);
            return true;
        }
        return fail("unexpected character");
    }
};

bool get_int(const JVal& o, const char* k, int64_t& out, bool required, int64_t dflt,
             std::string& err) {
    const JVal* v = o.get(k);
    if (!v) {
        if (required) { err = std::string("missing field '") + k + "'"; return false; }
        out = dflt;
        return true;
    }
    if (v->kind != JVal::NUM || v->num != (double)(int64_t)v->num) {
        err = std::string("field '") + k + "' is not an integer";
        return false;
    }
    out = (int64_t)v->num;
    return true;
}

}  // namespace

bool parse_tile_table(const std::string& text, TileTable& out, std::string& err) {
    Parser ps(text);
    JVal root;
    if (!ps.value(root, 0)) { err = ps.err; return false; }
    ps.ws();
    if (ps.i != text.size()) { err = "trailing characters after JSON value"; return false; }
    if (root.kind != JVal::OBJ) { err = "top level is not an object"; return false; }
    const JVal* entries = root.get("entries");
    if (!entries || entries->kind != JVal::ARR) { err = "missing 'entries' array"; return false; }
    TileTable t;
    for (const JVal& e : entries->arr) {
        if (e.kind != JVal::OBJ) { err = "entry is not an object"; return false; }
        int64_t N, K;
        if (!get_int(e, "N", N, true, 0, err) || !get_int(e, "K", K, true, 0, err)) return false;
        const JVal* dt = e.get("dtype");
        if (!dt || dt->kind != JVal::STR) { err = "missing 'dtype'"; return false; }
        int qtype;
        if (dt->str == "fp8_w8a8") qtype = 0;
        else if (dt->str == "int8_w8a8") qtype = 1;
        else { err = "unknown dtype '" + dt->str + "'"; return false; }
        int wlayout = 0;
        if (const JVal* wl = e.get("w_layout")) {
            if (wl->kind != JVal::STR) { err = "'w_layout' is not a string"; return false; }
            if (wl->str == "row_major") wlayout = 0;
            else if (wl->str == "packed16") wlayout = 1;
            else { err = "unknown w_layout '" + wl->str + "'"; return false; }
        }
        int sfmt = 0;
        if (const JVal* sf = e.get("scales")) {
            if (sf->kind != JVal::STR) { err = "'scales' is not a string"; return false; }
            if (sf->str == "fp32") sfmt = 0;
            else if (sf->str == "ue8m0") sfmt = 1;
            else { err = "unknown scales '" + sf->str + "'"; return false; }
        }
        const JVal* bs = e.get("block_shape");
        if (bs) {
            const bool two = bs->kind == JVal::ARR && bs->arr.size() == 2;
            const bool block = two && bs->arr[0].num == 128 && bs->arr[1].num == 128;
            // [1, K]: per-token x per-channel scales (a kernel family of its own)
            const bool channel = two && bs->arr[0].num == 1 && bs->arr[1].num == (double)K;
            if (!block && !channel) {
                err = "block_shape must be [128, 128] or [1, K]";
                return false;
            }
            if (channel) {
                if (sfmt != 0) { err = "'scales' does not apply to block_shape [1, K]"; return false; }
                sfmt = 2;
            }
        }
        const JVal* cfgs = e.get("configs");
        if (!cfgs || cfgs->kind != JVal::OBJ) { err = "missing 'configs' object"; return false; }
        std::map<int64_t, bfq_tile> buckets;
        for (auto& kv : cfgs->obj) {
            char* endp = nullptr;
            long long m = std::strtoll(kv.first.c_str(), &endp, 10);
            if (endp == kv.first.c_str() || *endp != '\0' || m <= 0) {
                err = "config key '" + kv.first + "' is not a positive integer";
                return false;
            }
            if (kv.second.kind != JVal::OBJ) { err = "config is not an object"; return false; }
            int64_t f[10];
            const char* names[10] = {"variant", "bm", "bn", "split_k", "waves_m", "waves_n",
                                     "stages", "group_m", "sched", "raster"};
            const int64_t dflt[10] = {0, 0, 0, 1, 1, 1, 2, 1, 0, 0};
            const bool req[10] = {true, true, true, false, true, true, false, false, false, false};
            for (int j = 0; j < 10; ++j)
                if (!get_int(kv.second, names[j], f[j], req[j], dflt[j], err)) return false;
            bfq_tile tl{};
            tl.variant = (int32_t)f[0];
            tl.bm = (int32_t)f[1];
            tl.bn = (int32_t)f[2];
            tl.bk = 128;
            tl.split_k = (int32_t)f[3];
            tl.waves_m = (int32_t)f[4];
            tl.waves_n = (int32_t)f[5];
            tl.stages = (int32_t)f[6];
            tl.group_m = (int32_t)f[7];
            tl.sched = (int32_t)f[8];
            tl.raster = (int32_t)f[9];
            buckets[(int64_t)m] = tl;
        }
        if (buckets.empty()) { err = "entry has no configs"; return false; }
        int64_t E = 0;
        if (e.get("E") && !get_int(e, "E", E, true, 0, err)) return false;
        if (E < 0 || E > 1023) { err = "'E' must be in [0, 1023]"; return false; }
        if (E > 0 && sfmt == 2) { err = "grouped (E > 0) entries take block scales"; return false; }
        t.entries[TableKey{N, K, qtype, wlayout, sfmt, E}] = std::move(buckets);
    }
    out = std::move(t);
    return true;
}

int64_t nearest_bucket(const std::map<int64_t, bfq_tile>& buckets, int64_t M) {
    int64_t best = buckets.begin()->first;
    for (auto& kv : buckets) {            // ascending keys: a tie keeps the smaller one
        int64_t d = kv.first > M ? kv.first - M : M - kv.first;
        int64_t db = best > M ? best - M : M - best;
        if (d < db) best = kv.first;
    }
    return best;
}

}  // namespace bfq
