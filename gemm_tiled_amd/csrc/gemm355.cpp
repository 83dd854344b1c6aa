// gemm355.cpp -- host side of libgemm355: argument checks, the special
// cases, tile selection (pin > tuned > heuristic), the f16r workspace, the
// per-shape autotuner and its cache, and the exported C ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cctype>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "gemm355.h"
#include "internal.hpp"
#include "workspace.hpp"

namespace g355 {
namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1024;   // kernels index tiles with int

// ---------------------------------------------------------------------------
// Logging (GEMM355_LOG=debug prints every choice of tile and path).
// ---------------------------------------------------------------------------
bool log_debug() {
    static const bool on = [] {
        const char* v = std::getenv("GEMM355_LOG");
        return v && (std::strcmp(v, "debug") == 0 || std::strcmp(v, "1") == 0);
    }();
    return on;
}

const char* mode_name(int mode) { return mode == GEMM355_MODE_F32 ? "f32" : "f16r"; }

// Up to this many rows of C the heuristic picks the few-rows configuration,
// then the f32-panel ring where it takes the shape (f16r: up to kRingRows, or
// twice that when N x K is at most 2^22; f32: up to kPanelRowsF32, or four
// times that when N x K is at most 2^21: 1024^3 in 26 us against 29 us on the
// best tile that does not split K), else in
// the f16r mode the register-staged configuration that rounds on load up to
// kDirectRows, and up to kSplitKRows the split-K configuration.
constexpr int64_t kRowsRows = 16;
constexpr int64_t kRingRows = 512;
constexpr int64_t kPanelRowsF32 = 256;
constexpr int64_t kDirectRows = 384;
constexpr int64_t kSplitKRows = 128;
// Compute units of the MI355X (gfx950).
constexpr int64_t kCUs = 256;
// Workgroups a split-K launch aims for (three per CU), the least k per slice,
// and the most bytes its partial tiles may take in the workspace.
constexpr int64_t kSplitKTarget = 3 * kCUs;
constexpr int64_t kSplitKMinDepth = 128;
constexpr int64_t kSplitKMaxBytes = int64_t{1} << 30;
// Least run of a stream-K f32 ring call (16-deep panels), and the panels its
// partial sums are counted as in the choice of the run.
constexpr int64_t kRingMinPanels = 32;
constexpr int64_t kRingSkOverhead = 12;
// Least k per slice of the KS=3 configurations.
constexpr int64_t kDirectMinDepth = 512;
// Most workgroups (of four waves) a few-rows launch splits K into.
constexpr int64_t kRowsMaxWgs = 8 * kCUs;

// ---------------------------------------------------------------------------
// Instances and configuration strings.
// ---------------------------------------------------------------------------
std::vector<TileConfig> configs_of(int mode) {
    std::vector<TileConfig> out;
    int n = 0;
    if (mode == GEMM355_MODE_F32) {
        const F32Instance* t = f32_instances(&n);
        for (int i = 0; i < n; ++i) out.push_back(t[i].cfg);
    } else {
        const F16Instance* t = f16_instances(&n);
        for (int i = 0; i < n; ++i) out.push_back(t[i].cfg);
        const DirectInstance* d = direct_instances(&n);
        for (int i = 0; i < n; ++i) out.push_back(d[i].cfg);
    }
    const DirectInstance* d = panel_ring_instances(mode, &n);
    for (int i = 0; i < n; ++i) out.push_back(d[i].cfg);
    out.push_back(splitk_config(mode));
    out.push_back(rows_config(mode));
    return out;
}

std::string format_config(const TileConfig& c) {
    char b[128];
    std::snprintf(b, sizeof b, "BM=%d BN=%d BK=%d ST=%d WM=%d WN=%d GM=%d", c.bm, c.bn, c.bk,
                  c.st, c.wm, c.wn, c.gm);
    std::string out = b;
    if (c.ks) out += " KS=" + std::to_string(c.ks);
    return out;
}

// Parse "KEY=VALUE ..." into the first compiled instance matching every given
// key.  Returns false on a syntax error, an unknown key or no match.
bool parse_config(int mode, const char* spec, TileConfig* out) {
    // bm bn bk wm wn gm st ks; an absent key matches any value, except KS,
    // whose absence means the configurations without split-K (KS = 0)
    int want[8] = {-1, -1, -1, -1, -1, -1, -1, 0};
    const char* p = spec;
    bool any = false;
    while (*p) {
        while (*p && std::isspace(static_cast<unsigned char>(*p))) ++p;
        if (!*p) break;
        const char* k0 = p;
        while (*p && *p != '=' && !std::isspace(static_cast<unsigned char>(*p))) ++p;
        if (*p != '=') return false;
        std::string key(k0, p - k0);
        ++p;
        char* end = nullptr;
        const long v = std::strtol(p, &end, 10);
        if (end == p || v < 0 || v > 4096) return false;
        if (*end && !std::isspace(static_cast<unsigned char>(*end))) return false;
        p = end;
        for (auto& ch : key) ch = static_cast<char>(std::toupper(static_cast<unsigned char>(ch)));
        int slot = -1;
        if (key == "BM" || key == "TILE_M") slot = 0;
        else if (key == "BN" || key == "TILE_N") slot = 1;
        else if (key == "BK" || key == "TILE_K") slot = 2;
        else if (key == "WM") slot = 3;
        else if (key == "WN") slot = 4;
        else if (key == "GM") slot = 5;
        else if (key == "ST" || key == "STAGES") slot = 6;
        else if (key == "KS" || key == "SPLITK") slot = 7;
        if (slot < 0 || (v == 0 && slot != 7)) return false;
        want[slot] = static_cast<int>(v);
        any = true;
    }
    if (!any) return false;
    for (const TileConfig& c : configs_of(mode)) {
        const int have[8] = {c.bm, c.bn, c.bk, c.wm, c.wn, c.gm, c.st, c.ks};
        bool ok = true;
        for (int i = 0; i < 8; ++i)
            if (want[i] >= 0 && want[i] != have[i]) ok = false;
        if (ok) {
            *out = c;
            return true;
        }
    }
    return false;
}

// ---------------------------------------------------------------------------
// Pins, tuned cache.
// ---------------------------------------------------------------------------
struct Key {
    int mode;
    int64_t M, N, K;
    int vec_a, vec_b, beta0;
    int trans;   // operand layouts: bit 0 op(A) = A^T, bit 1 op(B) = B^T
    bool operator<(const Key& o) const {
        return std::tie(mode, M, N, K, vec_a, vec_b, beta0, trans) <
               std::tie(o.mode, o.M, o.N, o.K, o.vec_a, o.vec_b, o.beta0, o.trans);
    }
};

// The cache and log name of a mode and layout: "f32", "f32:TN" (op(A) = A^T),
// "f16r:NT" (op(B) = B^T), ...
std::string layout_name(int mode, int trans) {
    std::string s = mode == GEMM355_MODE_F32 ? "f32" : "f16r";
    if (trans) {
        s += ':';
        s += (trans & 1) ? 'T' : 'N';
        s += (trans & 2) ? 'T' : 'N';
    }
    return s;
}

struct State {
    std::mutex mu;
    bool env_read = false;
    bool pin_set[2] = {false, false};
    bool pin_bad[2] = {false, false};   // an invalid pin from the environment
    TileConfig pin[2];
    std::map<Key, TileConfig> cache;
    std::string cache_path;
};

State& state() {
    static State s;
    return s;
}

size_t load_cache_locked(State& st, const char* path);

void read_env_locked(State& st) {
    if (st.env_read) return;
    st.env_read = true;
    const char* names[2] = {"GEMM355_CONFIG_F32", "GEMM355_CONFIG_F16R"};
    for (int m = 0; m < 2; ++m) {
        const char* v = std::getenv(names[m]);
        if (!v || !*v) continue;
        TileConfig c;
        if (parse_config(m, v, &c)) {
            st.pin[m] = c;
            st.pin_set[m] = true;
        } else {
            st.pin_bad[m] = true;
            std::fprintf(stderr, "[gemm355] %s=\"%s\" names no compiled configuration\n",
                         names[m], v);
        }
    }
    const char* path = std::getenv("GEMM355_TUNE_CACHE");
    if (path && *path) {
        st.cache_path = path;
        load_cache_locked(st, path);
    }
}

bool vec_ok(const float* p, int64_t ld) {
    return (ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(p) & 15) == 0);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// The ring configurations -- f32 (direct-to-LDS copies, BK = 16, three or
// more stages) and f16r half-depth (BK = 32) -- and their stream-K form: when
// whole rounds of tiles would leave resident slots idle, the slots take the
// whole rounds they can fill (data-parallel, in the usual tile order) and
// then the (tile, panel) units of the remaining tiles in equal runs of at
// least kRingMinPanels units, if that beats the whole rounds by 5% counting
// kRingSkOverhead panels for the split tiles' partial sums.  Runs that start
// at different depths of their tiles share no operand panels in the cache,
// which is why the remaining tiles alone are dealt this way.
// What the f32 ring can take of a call: nothing (leading dimensions too large
// for the masked copies' 32-bit offsets: up to 256 stored rows of a panel of
// an operand whose k runs along its rows, 16 of one whose k runs down them),
// any shape through its masked form, or also whole tiles unmasked (16-byte
// aligned rows); and the operand layouts (bit 0 op(A) = A^T, bit 1 op(B) =
// B^T).
struct RingRows {
    enum Kind { None, Any, Aligned };
    Kind kind = None;
    int trans = 0;
    bool none() const { return kind == None; }
    bool aligned() const { return kind == Aligned; }
};
RingRows ring_rows(int trans, const float* A, int64_t lda, const float* B, int64_t ldb) {
    const int64_t a_lim = (trans & 1) ? int64_t{1} << 24 : int64_t{1} << 20;
    const int64_t b_lim = (trans & 2) ? int64_t{1} << 20 : int64_t{1} << 24;
    if (lda >= a_lim || ldb >= b_lim) return RingRows{RingRows::None, trans};
    return RingRows{vec_ok(A, lda) && vec_ok(B, ldb) ? RingRows::Aligned : RingRows::Any, trans};
}
// The masked ring's rate relative to the unmasked one (4-byte copies, edge
// tiles), with the reuse constant kReuseF32 of whole_cost and the strips'
// efficiency kStripRate fitted to every f32 configuration timed pinned at 29
// shapes from 512 x 4096^2 to 6144^3, 15 of them ragged (1000^3 to 6000^3,
// 4000 x 4097 x 4093), so that every timed configuration kept its plan (whole
// call, or block and strips) and the pick came within 2.2% of the fastest at
// all but 1000^3 (4.6%) and 3500^3 (3.7%).
constexpr double kRingMaskedRate = 0.93;
constexpr double kReuseF32 = 10.0;
constexpr double kStripRate = 0.95;
// The masked ring with 16-byte copies (16-byte aligned rows, N and K multiples
// of 4): 4088^3 in 951 us against 939 us for 4096^3, 2-3% below the unmasked
// ring per flop (the 4-byte copies: 1019 us).
constexpr double kRingWideRate = 0.98;

bool is_f32_ring(const TileConfig& c) {
    return c.mode == GEMM355_MODE_F32 && c.bk == 16 && c.st >= 3 && c.ks == 0;
}
bool is_f16_ring(const TileConfig& c) {
    return c.mode == GEMM355_MODE_F16R && c.bk == 32 && c.ks == 0;
}

struct RingSk {
    int64_t q = 0, dp = 0, grid = 0;   // q = 0: one tile per workgroup
    double panels = 0;                 // estimated panels per slot
};

RingSk ring_sk(const TileConfig& c, int64_t M, int64_t N, int64_t K) {
    RingSk out;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t nkt = c.mode == GEMM355_MODE_F32 ? (K + 15) / 16 : round_up(K, 64) / 32;
    // LDS of one workgroup: NS stages of BM x BK A rows and BK x BN B values
    // (f32 B rows padded by 16 bytes), binary16 or f32
    const int64_t lds = c.mode == GEMM355_MODE_F32
                            ? int64_t{c.st} * (c.bm * 64 + 16 * (c.bn * 4 + 16))
                            : int64_t{c.st} * (c.bm + c.bn) * 64;
    const int64_t slots = kCUs * std::max<int64_t>(1, (160 * 1024) / lds);
    const int64_t whole = (tiles + slots - 1) / slots * nkt;
    out.panels = static_cast<double>(whole);
    if (tiles % slots == 0 || tiles * nkt >= (int64_t{1} << 31)) return out;
    // a binary16 ring with 128 x 128 wave tiles has no stream-K form
    if (c.mode == GEMM355_MODE_F16R && (c.bm / c.wm) * (c.bn / c.wn) >= 128 * 128) return out;
    const int64_t dp = tiles / slots;
    // In binary16 the runs start at different depths, so no two share operand
    // panels in the cache and that phase is bound by memory: measured worse
    // than whole rounds once the tiles left after them fill more than a
    // quarter of the slots (3072^3 on 256^2 tiles, 144 of 256 slots and no
    // whole round: 134 us against 88 us; 5120^3, one round and 144 tiles
    // left: 356 against 283 us), better below (2048 x 2048 x 8192, 64 tiles:
    // 131 against 172 us; 6144^3, two rounds and 64 tiles left: 455 against
    // 529 us on the 256^2 panels).  With no whole round the call is counted at
    // twice its panels.
    const bool f16_alone = c.mode == GEMM355_MODE_F16R && dp == 0;
    if (c.mode == GEMM355_MODE_F16R && (tiles - dp * slots) * 4 > slots) return out;
    const int64_t rest = (tiles - dp * slots) * nkt;
    const int64_t q = std::max<int64_t>((rest + slots - 1) / slots, kRingMinPanels);
    const double panels = static_cast<double>(dp * nkt + q + kRingSkOverhead) * (f16_alone ? 2 : 1);
    if (panels >= 0.95 * static_cast<double>(whole)) return out;
    const int64_t grid = dp > 0 ? slots : (rest + q - 1) / q;
    if (grid * 2 * c.bm * c.bn * 4 > kSplitKMaxBytes) return out;
    out.q = q;
    out.dp = dp;
    out.grid = grid;
    out.panels = panels;
    return out;
}

// The rate of an f16r configuration's tile on a CU relative to the 256^2
// half-depth ring with eight waves, fitted (with the rest of the f16r cost
// in whole_cost) to timings: 256^2 with four waves 0.85, 256 x 128 and
// 128 x 256 with eight 0.93, 128^2 (two workgroups per CU) with four 0.86
// and with eight 0.87 on a grid of at most one round (512 tiles), 0.85 on a
// larger one (eight waves 0.6-7% faster at 9 of 10 shapes of 100-256 tiles,
// the tenth even, 0.4-1.3% slower at 4 of 5 of 676-3025).  Others by their
// reuse r = BM BN / (BM + BN) as r / (r + 85) against the 256^2 tile's, the
// full-depth panels at 1 / 1.2 of that (the half-depth ring at a tile ran
// 1.1-1.4 times faster).
double f16_efficiency(const TileConfig& c, double tiles) {
    const int waves = c.wm * c.wn;
    if (is_f16_ring(c)) {
        if (c.bm == 256 && c.bn == 256) return waves == 8 ? 1.0 : 0.85;
        if (c.bm * c.bn == 256 * 128 && waves == 8) return 0.93;
        if (c.bm == 128 && c.bn == 128) return waves != 8 ? 0.86 : tiles <= 512 ? 0.87 : 0.85;
    }
    const double r = static_cast<double>(c.bm) * c.bn / (c.bm + c.bn);
    const double rel = (r / (r + 85.0)) / (128.0 / (128.0 + 85.0));
    return is_f16_ring(c) ? rel : rel / 1.2;
}

// Estimated time of configuration c on an M x N x K call run whole
// (arbitrary units): rounds of workgroups over 256 CUs (two per CU for tiles
// under 256 x 128) times the work of a tile, over the reuse efficiency r /
// (r + kReuseF32) of the tile, r = BM BN / (BM + BN).  An f32 ring call deals its
// work in equal runs when whole rounds would leave CUs idle (stream-K,
// counted by the panels of a slot plus the partial sums' overhead) and stages
// its panels faster than the register-staged kernel (10-20% measured, counted
// as 20%), the masked form at kRingMaskedRate of that (kRingWideRate with
// 16-byte copies).
double whole_cost(const TileConfig& c, int64_t M, int64_t N, int64_t K, RingRows rows) {
    const bool ring = is_f32_ring(c) && !rows.none();
    const bool whole = rows.aligned() && M % c.bm == 0 && N % c.bn == 0 && K % 16 == 0;
    const double tiles = static_cast<double>((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const double per_cu = (c.bm * c.bn >= 256 * 128) ? 1.0 : 2.0;
    const RingSk sk = ring || is_f16_ring(c) ? ring_sk(c, M, N, K) : RingSk{};
    const double kpad = static_cast<double>(round_up(K, c.bk));
    const double rounds = sk.q > 0 ? sk.panels / (kpad / c.bk) : std::ceil(tiles / (256.0 * per_cu));
    const double reuse = static_cast<double>(c.bm) * c.bn / (c.bm + c.bn);   // flop per loaded element
    if (c.mode == GEMM355_MODE_F16R) {
        // f16r: the time of the busiest CU.  Whole rounds of 256 tiles count
        // one tile each; a part-filled last round of L tiles counts
        // (L / 256)^0.4 of one, since a chip with idle CUs runs each tile
        // faster (less contention for power, cache and memory: 64 256^2 tiles
        // ran each at 0.4 of a full round's time, 128 at 0.7).  A stream-K
        // call counts its panels per slot, the panels of the runs 2.5 times
        // (runs at different depths share no operand panels in the cache, so
        // that phase is bound by memory).  A tile's time is its work over the
        // efficiency of its configuration (f16_efficiency).  Fitted to the
        // ring configurations timed pinned at 43 shapes from 768 x 4096^2 to
        // 8192^3, 15 of them ragged: the pick within 2.4% of the fastest at
        // all but 2048^3 (3%) and 7000^3 (4.2%).
        const double t_tile = c.bm * c.bn * kpad / f16_efficiency(c, tiles);
        if (sk.q > 0) {
            // in runs the 256^2 tile with 2 x 4 waves was 1-5% faster than
            // with 4 x 2 (6144^3 448 against 469 us; the stream-K form of the
            // 4 x 2 tile spills registers), in whole rounds 1-4% slower
            // (8192^2 x 2048 272 against 262)
            const double slots_per_cu =
                std::max(1.0, std::floor(160.0 * 1024 / (static_cast<double>(c.st) * (c.bm + c.bn) * 64)));
            const double waves = (c.bm == 256 && c.bn == 256 && c.wm == 4) ? 1.03 : 1.0;
            const double nkt = kpad / c.bk;
            const double panels = (static_cast<double>(sk.dp) * nkt +
                                   2.5 * static_cast<double>(sk.q + kRingSkOverhead)) *
                                  (sk.dp == 0 ? 2.0 : 1.0);
            return slots_per_cu * panels / nkt * t_tile * waves;
        }
        const double full = std::floor(tiles / 256.0), left = tiles - 256.0 * full;
        return (full + std::pow(left / 256.0, 0.4)) * t_tile;
    }
    // 16-byte masked copies: along each operand's contiguous dimension a
    // multiple of 4 elements
    const int64_t a_run = (rows.trans & 1) ? M : K, b_run = (rows.trans & 2) ? K : N;
    const bool wide = rows.aligned() && a_run % 4 == 0 && b_run % 4 == 0;
    const double eff = reuse / (reuse + kReuseF32) *
                       (ring ? 1.2 * (whole ? 1.0 : wide ? kRingWideRate : kRingMaskedRate) : 1.0);
    return rounds * per_cu * c.bm * c.bn * kpad / eff;
}

// The configuration of a strip left over by a split ring call (RingBlock):
// the few-rows one for up to 16 rows or (in its few-columns form) 16 columns,
// split-K tiles for another thin strip (a strip of few columns is a long K
// loop per tile, so it needs K split), else the
// register-staged 64 x 64 tile.  Its cost in the units of whole_cost: a thin
// strip its share of the chip's rounds, a wide one whole rounds of 64 x 64
// tiles, at the efficiency kStripRate.
TileConfig strip_config(int mode, int64_t rows, int64_t cols) {
    if (rows <= kRowsRows || cols <= kRowsRows) return rows_config(mode);
    if (rows <= 128 || cols <= 128) return splitk_config(mode);
    TileConfig edge;
    parse_config(mode, "BM=64 BN=64 BK=16 ST=2", &edge);
    return edge;
}
double strip_cost(int64_t rows, int64_t cols, int64_t k) {
    const double tiles = static_cast<double>((rows + 63) / 64) * ((cols + 63) / 64);
    const double rounds = rows <= 128 || cols <= 128 ? tiles / 512.0 : std::ceil(tiles / 512.0);
    return rounds * 2.0 * 64 * 64 * static_cast<double>(round_up(k, 16)) / kStripRate;
}

// The part of a ragged call that an f32 ring configuration runs itself: the
// block [0, mb) x [0, nb) of C over k in [0, kb); the right strip [0, M) x
// [nb, N), the bottom strip [mb, M) x [0, nb) and the k tail of the block go
// to strip configurations.  Candidates: the whole call (masked ring, or the
// unmasked one on whole tiles), the call without its last partial tile row,
// column or both (that partial tile can cost a whole extra round or a share
// of stream-K runs), and with 16-byte aligned rows the block of whole tiles
// over K rounded down to 16 (the unmasked ring).  The cheapest by whole_cost
// + strip_cost wins, the whole call on a near tie.
struct RingBlock {
    int64_t mb, nb, kb;
    double cost;
};
RingBlock ring_block(const TileConfig& c, RingRows rows, int64_t M, int64_t N, int64_t K) {
    RingBlock best{M, N, K, whole_cost(c, M, N, K, rows)};
    // (the block and strips address the operands as stored: plain layout only)
    if (!is_f32_ring(c) || rows.none() || rows.trans != 0) return best;
    const int64_t M0 = M / c.bm * c.bm, N0 = N / c.bn * c.bn, K16 = K / 16 * 16;
    auto consider = [&](int64_t mb, int64_t nb, int64_t kb) {
        if (mb <= 0 || nb <= 0 || kb <= 0 || (mb == M && nb == N && kb == K)) return;
        double cost = whole_cost(c, mb, nb, kb, rows);
        if (nb < N) cost += strip_cost(M, N - nb, K);
        if (mb < M) cost += strip_cost(M - mb, nb, K);
        if (kb < K) cost += strip_cost(mb, nb, K - kb);
        if (cost < 0.99 * best.cost) best = RingBlock{mb, nb, kb, cost};
    };
    consider(M0, N, K);
    consider(M, N0, K);
    consider(M0, N0, K);
    if (rows.aligned()) consider(M0, N0, K16);
    return best;
}

double estimated_cost(const TileConfig& c, int64_t M, int64_t N, int64_t K, RingRows rows) {
    return ring_block(c, rows, M, N, K).cost;
}

// The grid of a KS=3 launch: its tiles, the workgroups a CU holds at once
// (the LDS of the stages, at most four waves per SIMD), and K in slices, each
// at least kDirectMinDepth deep (a multiple of the panel depth), the partial
// tiles within kSplitKMaxBytes.  Up to `reach` slices would take the grid to
// one round of resident workgroups; of 1..reach the count taken is the one
// that loads the busiest CU least (workgroups a CU x slice depth), on a tie
// the fewer slices where one workgroup fills a CU and the more where several
// share one (they hide each other's latency).  A grid of one-workgroup tiles
// that cannot fill the CUs evenly so runs as one round of deeper slices
// rather than a full round and a part-filled second one: f16r 128^2,
// 1536^2 x 1024 (144 tiles) and 1792^2 x 1024 (196) in 18.7 and 20.0 us
// against 25.9 and 28.6 on 288 and 392 workgroups of half depth; 128 x 256 at
// 1280^2 x 4096 (50 tiles) 37.4 on 5 slices against 48.3 on 6.  f32 64 x 128
// (two workgroups a CU) at 768 x 4096^2 keeps its 768 workgroups: on 384 it
// ran in 260 us against 207.
struct DirectGrid {
    int64_t tiles_m, tiles_n, per_cu, slices, depth, reach;
};
DirectGrid direct_grid(const TileConfig& cfg, int64_t M, int64_t N, int64_t K) {
    DirectGrid d{};
    d.tiles_m = (M + cfg.bm - 1) / cfg.bm;
    d.tiles_n = (N + cfg.bn - 1) / cfg.bn;
    const int64_t tiles = d.tiles_m * d.tiles_n;
    const int64_t lds_bytes = cfg.bk == 32 ? int64_t{cfg.st} * (cfg.bm * 128 + 32 * cfg.bn * 4)
                                           : 2 * int64_t{cfg.bm + cfg.bn} * 128;
    d.per_cu = std::max<int64_t>(1, std::min<int64_t>((160 * 1024) / lds_bytes, 4 * 4 / (cfg.wm * cfg.wn)));
    const int64_t tile_bytes = int64_t{cfg.bm} * cfg.bn * 4;
    const int64_t round = kCUs * d.per_cu;   // resident workgroups
    int64_t reach = std::max<int64_t>(1, (round + tiles - 1) / tiles);
    reach = std::min(reach, std::max<int64_t>(1, K / kDirectMinDepth));
    reach = std::min(reach, std::max<int64_t>(1, kSplitKMaxBytes / (tiles * tile_bytes)));
    d.reach = reach;
    int64_t slices = 1;
    for (int64_t s = 2; s <= reach; ++s) {   // busiest CU, K as the unit: ceil(tiles s / CUs) / s
        const int64_t load_s = (tiles * s + kCUs - 1) / kCUs * slices;
        const int64_t load_best = (tiles * slices + kCUs - 1) / kCUs * s;
        if (load_s < load_best || (load_s == load_best && d.per_cu > 1)) slices = s;
    }
    d.depth = round_up((K + slices - 1) / slices, cfg.bk);
    d.slices = (K + d.depth - 1) / d.depth;
    return d;
}

// The f32-panel ring configuration (KS=3, BK=32) for a call whose shape that
// ring takes: the tile by the rows of C, measured best at N = K = 4096 --
// f16r: 32 x 64 up to 64 rows, 64 x 64 up to 160, 128 x 128 up to 256,
// 128 x 256 beyond; f32: 32 x 128 up to 32 rows, 64 x 64 up to 128, 64 x 128
// beyond -- then a smaller tile of the mode's ladder while the call's
// workgroups (tiles x the most K slices it could take, the reach of
// direct_grid) would not fill one round of the CUs (f16r) or
// half a round (f32: there 32 x 128 at 17 rows, 256 workgroups, beat 32 x 64
// with 512, 21 against 27 us, while f16r's 1024^3 took 64 x 64 at 13 us over
// 128 x 128's half round at 16 us).
TileConfig panel_ring_config(int mode, int64_t M, int64_t N, int64_t K) {
    static const char* const kF16r[] = {
        "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 GM=8 KS=3", "BM=64 BN=64 BK=32 ST=4 WM=4 WN=1 GM=8 KS=3",
        "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3", "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 GM=8 KS=3"};
    static const char* const kF32[] = {
        "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 GM=8 KS=3", "BM=32 BN=128 BK=32 ST=4 WM=2 WN=2 GM=8 KS=3",
        "BM=64 BN=64 BK=32 ST=4 WM=4 WN=1 GM=8 KS=3", "BM=64 BN=128 BK=32 ST=3 WM=2 WN=2 GM=8 KS=3"};
    const bool f32 = mode == GEMM355_MODE_F32;
    const char* const* ladder = f32 ? kF32 : kF16r;
    int i = f32 ? (M <= 32 ? 1 : M <= 128 ? 2 : 3) : (M <= 64 ? 0 : M <= 160 ? 1 : M <= 256 ? 2 : 3);
    const int64_t fill = f32 ? 2 : 1;   // workgroups x fill >= one round
    TileConfig c{};
    for (; i >= 0; --i) {
        parse_config(mode, ladder[i], &c);
        const DirectGrid d = direct_grid(c, M, N, K);
        // f16r 128 x 256 in 6 or more slices: the last workgroup of a tile
        // adds many large partial tiles alone, so 128^2 is taken -- 1.11-1.49
        // times faster at 7 shapes (512 x 1024 x 8192, 16 slices, 49.9 us
        // against 33.5; 1024^2 x 4096, 8, 33.6 against 29.5; 640 x 2048 x
        // 4096, 6, 32.5 against 28.3), 3% slower at 1024^2 x 8192; from 5
        // slices 128^2 has too few workgroups (384 x 4096^2 35.8 against 39.8)
        if (!f32 && c.bn == 256 && d.slices > 5) continue;
        if (fill * d.tiles_m * d.tiles_n * d.reach >= kCUs * d.per_cu) break;
    }
    return c;
}

// Heuristic when nothing is pinned or tuned: estimate the time of each
// instance as (rounds of workgroups over 256 CUs) x (work per tile) / (reuse
// efficiency of the tile), the trade-off of the phobos "Tuning" section:
// larger tiles reuse more, but leave fewer workgroups to fill the chip.
TileConfig heuristic(int mode, int64_t M, int64_t N, int64_t K, RingRows rows) {
    // (the f32-panel ring: 16-byte aligned rows, K % 32 == 0, and a multiple
    // of 4 along B's rows as stored K x N and along A's as stored K x M)
    const bool panels = rows.aligned() && K % 32 == 0 && ((rows.trans & 2) || N % 4 == 0) &&
                        (!(rows.trans & 1) || M % 4 == 0);
    // a few rows of C (memory-bound, too few tiles): the few-rows
    // configuration up to one 16-row group, then the split-K tiles.  With B
    // stored N x K the few-rows kernel's register layout reads B^T 16 stored
    // rows per load, while the f32-panel ring copies whole 128-byte pieces of
    // rows into its panels: at K = N = 4096 and 1 to 16 rows the ring on 16 x
    // 128 tiles ran f16r in 15.9-16.2 us against 19.3-21.9, f32 in 18.2-18.5
    // against 19.3-20.6 (on 32 x 128 tiles 16.3-16.9 and 18.9-19.6).
    if (M <= kRowsRows) {
        TileConfig ring;
        if ((rows.trans & 2) && panels && N >= 128 &&
            parse_config(mode, "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 GM=8 KS=3", &ring))
            return ring;
        return rows_config(mode);
    }
    // A few columns of C (measured at M = K = 4096): in f32 the same
    // configuration on the transposed problem up to 16 columns (4096 x 16 x
    // 4096 in 20 us against 81 us on the masked 128 x 256 ring, 8192 x 1 x
    // 8192 in 46 against 283 us), then up to 64 columns the f32-panel ring on
    // 64 x 64 tiles (26 us); in f16r the transposed few-rows form for one or
    // two columns (18.5 us against 19.6) and from 4 to 64 columns the
    // f32-panel ring on 32 x 64 tiles (16 us against 21 on the transposed
    // form, 54 on the packed 64 x 64 tiles).
    if (N <= 64 && M >= 4 * N) {
        TileConfig thin;
        if (panels && mode == GEMM355_MODE_F16R && N >= 4 &&
            parse_config(mode, "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 GM=8 KS=3", &thin))
            return thin;
        // f32, at most 16 columns: the 16-row tile of the f32-panel ring on the
        // transposed problem (4096 x 4..16 x 4096 in 18.3-18.7 us against
        // 19.8-20.1 on the few-rows configuration's few-columns form), where
        // that takes it
        if (mode == GEMM355_MODE_F32 && N <= kRowsRows && !(rows.trans & 1) && rows.aligned() &&
            K % 32 == 0 && ((rows.trans & 2) || N % 4 == 0) &&
            parse_config(mode, "BM=16 BN=128 BK=32 ST=4 WM=1 WN=2 GM=8 KS=3", &thin))
            return thin;
        if (N <= kRowsRows) return rows_config(mode);
        if (panels && parse_config(mode, mode == GEMM355_MODE_F32
                                             ? "BM=64 BN=64 BK=32 ST=4 WM=4 WN=1 GM=8 KS=3"
                                             : "BM=32 BN=64 BK=32 ST=4 WM=2 WN=1 GM=8 KS=3",
                                   &thin))
            return thin;
    }
    if (N <= kRowsRows) return rows_config(mode);
    // (from 512 rows on the packed path wins once N x K is large: 768 x 4096^2
    // 60 us packed against 79 us on the ring, 1024 x 8192^2 193 against 220)
    // (and, measured, where the packed tiles are too few for a deep K, which
    // the ring splits over workgroups -- K >= 4096 with M N <= 2^21 and
    // min(M, N) <= 1280, or M, N <= 1536: 1024 x 2048 x 4096 39 us against
    // 56, 1280^2 x 4096 36 against 45, 1448^2 x 4096 43 against 46, 1536^2 x
    // 4096 42 against 44; not 1792^2 x 4096 (54 against 46 on the packed
    // path), 768 x 4096^2 (60 against 52) or 1800 x 1280 x 4096 (even)
    // -- or where K is so shallow that the packing pass dominates -- K <= 512
    // with M, N <= 2048: 2048^2 x 512 12.8 us against 18.8, 2048^2 x 256 8.5
    // against 15.2)
    const bool deep_few = K >= 4096 && ((M * N <= (int64_t{1} << 21) && std::min(M, N) <= 1280) ||
                                        std::max(M, N) <= 1536);
    if (panels && mode == GEMM355_MODE_F16R &&
        (M <= kRingRows || (M <= 2 * kRingRows && N * K <= (int64_t{1} << 22)) || deep_few ||
         (K <= 512 && M <= 2048 && N <= 2048)))
        return panel_ring_config(mode, M, N, K);
    // f16r, K = 513-2048: the 128^2 f32-panel ring where its grid, counted
    // in 1024-deep slices, fits one round of the CUs (each tile then runs
    // whole or in slices of at most 1024 in one round, with no packing pass):
    // 1.07-1.37 times the packed path's speed at 17 shapes, K = 640-1024 and
    // 100-256 tiles (1280^2 x 1024 16.2 us against 20.6, 2048^2 x 1024 21.9
    // against 26.4, 4096 x 1024^2 21.8 against 26.0), K = 1536-2048 and
    // 80-128 tiles (1280^2 x 2048 23.1 against 27.7).  Where a tile runs a
    // whole K of 2048 the packed path wins: 1792^2 x 2048 28.2 against 31.8,
    // 2048^2 x 2048 31.1 against 33.1.
    if (panels && mode == GEMM355_MODE_F16R && K > 512 && K <= 2048 &&
        ((M + 127) / 128) * ((N + 127) / 128) * ((K + 1023) / 1024) <= kCUs) {
        TileConfig c{};
        parse_config(mode, "BM=128 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3", &c);
        return c;
    }
    // (and at K = 513-1024 the 256 x 128 or 128 x 256 tile, its long side
    // along the longer of M and N, where that grid fits one round: 1.05-1.33
    // times the packed path's speed at 18 shapes, 2304^2 x 1024 28.0 us
    // against 29.3, 8192 x 1024^2 28.5 against 32.4, 2560^2 x 640 19.3
    // against 25.7; 3072^2 x 1024, 288 tiles, stays packed: 37 us against 50)
    if (panels && mode == GEMM355_MODE_F16R && K > 512 && K <= 1024 &&
        ((std::max(M, N) + 255) / 256) * ((std::min(M, N) + 127) / 128) <= kCUs) {
        TileConfig c{};
        parse_config(mode, M >= N ? "BM=256 BN=128 BK=32 ST=3 WM=4 WN=2 GM=8 KS=3"
                                  : "BM=128 BN=256 BK=32 ST=3 WM=2 WN=4 GM=8 KS=3", &c);
        return c;
    }
    if (panels && mode == GEMM355_MODE_F32 &&
        (M <= kPanelRowsF32 || (M <= 4 * kPanelRowsF32 && N * K <= (int64_t{1} << 21))))
        return panel_ring_config(mode, M, N, K);
    if (mode == GEMM355_MODE_F16R && M <= kDirectRows) {
        // rounding on load: no packing pass, whose cost grows with N x K
        const int bm = M <= 48 ? 32 : M <= 160 ? 64 : 128;
        int n = 0;
        const DirectInstance* d = direct_instances(&n);
        for (int i = 0; i < n; ++i)
            if (d[i].cfg.bm == bm && d[i].cfg.bn == (bm == 128 ? 128 : 64)) return d[i].cfg;
    }
    if (M <= kSplitKRows) return splitk_config(mode);
    const std::vector<TileConfig> all = configs_of(mode);
    double best = 1e300;
    TileConfig pick = all.front();
    for (const TileConfig& c : all) {
        if (c.ks) continue;
        const double cost = estimated_cost(c, M, N, K, rows);
        if (cost < best * 0.999) {
            best = cost;
            pick = c;
        }
    }
    return pick;
}

enum class Source { Pin, Tuned, Heuristic };

int select_config(int mode, int trans, int64_t M, int64_t N, int64_t K, const float* A,
                  int64_t lda, const float* B, int64_t ldb, float beta, TileConfig* out,
                  Source* src) {
    State& st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    read_env_locked(st);
    if (st.pin_bad[mode] && !st.pin_set[mode]) return GEMM355_ERR_CONFIG;
    if (st.pin_set[mode]) {
        *out = st.pin[mode];
        *src = Source::Pin;
        return 0;
    }
    const Key key{mode, M, N, K, vec_ok(A, lda), vec_ok(B, ldb), beta == 0.f, trans};
    auto it = st.cache.find(key);
    if (it != st.cache.end()) {
        *out = it->second;
        *src = Source::Tuned;
        return 0;
    }
    *out = heuristic(mode, M, N, K, ring_rows(trans, A, lda, B, ldb));
    *src = Source::Heuristic;
    return 0;
}

// ---------------------------------------------------------------------------
// Device scratch of a call: the packed binary16 operands of the f16r mode,
// the partial tiles of the configurations that split K over workgroups and
// their arrival counters.  The entry points that may allocate lease it from
// a pool per device (workspace.hpp: the lease lasts from the call's first
// request until its last launch is enqueued; growth is stream-ordered, the
// host never waits); gemm355_gemm_noalloc takes it from a fixed device array.
// Every call is first planned with a DryScratch (no launch), which records
// what it will ask for, so a failure to allocate, or a call larger than the
// fixed array, is reported before any kernel is enqueued.
// ---------------------------------------------------------------------------
int status_of(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int>(e); }

struct HipBackend {
    using Stream = hipStream_t;
    using Event = hipEvent_t;
    int alloc(void** p, size_t bytes, hipStream_t s) {
        const hipError_t e = hipMallocAsync(p, bytes, s);
        return e == hipErrorOutOfMemory ? GEMM355_ERR_ALLOC : status_of(e);
    }
    int release(void* p, hipStream_t s) { return status_of(hipFreeAsync(p, s)); }
    int zero_u32(unsigned* p, size_t n, hipStream_t s) {
        return status_of(launch_fill_u32(p, static_cast<int64_t>(n), 0u, s));
    }
    int event_create(hipEvent_t* e) {
        return status_of(hipEventCreateWithFlags(e, hipEventDisableTiming));
    }
    void event_destroy(hipEvent_t e) { (void)hipEventDestroy(e); }
    int record(hipEvent_t e, hipStream_t s) { return status_of(hipEventRecord(e, s)); }
    bool idle(hipEvent_t e) { return hipEventQuery(e) == hipSuccess; }
    // an error of the query counts as capturing: the call then only reuses
    // what its stream already holds and allocates nothing
    bool capturing(hipStream_t s) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        return hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone;
    }
};

// Slots kept per device (each as large as the largest call it served).
constexpr size_t kPoolSlots = 8;
using Pool = ScratchPool<HipBackend>;

Pool* pool_of(int dev) {
    static std::mutex mu;
    static std::map<int, Pool*> pools;     // never destroyed: calls may run until exit
    static HipBackend* backend = new HipBackend();
    std::lock_guard<std::mutex> lock(mu);
    Pool*& p = pools[dev];
    if (!p) p = new Pool(*backend, kPoolSlots);
    return p;
}

// The device a stream's work runs on (the current device for the null
// stream): scratch must live there, whichever device is current.
int device_of(hipStream_t s, int* dev) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(s, &d) == hipSuccess) {
        *dev = static_cast<int>(d);
        return 0;
    }
    return status_of(hipGetDevice(dev));
}

class Scratch {
public:
    virtual ~Scratch() = default;
    // A buffer of at least `bytes` bytes and n zeroed arrival counters for
    // the launches of this call; 0 or a status.
    virtual int workspace(size_t bytes, void** out) = 0;
    virtual int counters(size_t n, unsigned** out) = 0;
    // Planning pass: the launch functions return right before launching.
    bool dry() const { return dry_; }
    // Obtain, before anything is launched, what a dry pass recorded.
    virtual int reserve(size_t bytes, size_t n) {
        void* w = nullptr;
        unsigned* c = nullptr;
        int rc = bytes ? workspace(bytes, &w) : 0;
        if (rc == 0 && n) rc = counters(n, &c);
        return rc;
    }

protected:
    bool dry_ = false;
};

// Records the largest requests of a call; hands out a stand-in pointer that
// no kernel ever sees (nothing is launched in a dry pass).
class DryScratch : public Scratch {
public:
    DryScratch() { dry_ = true; }
    int workspace(size_t bytes, void** out) override {
        ws = std::max(ws, bytes);
        *out = reinterpret_cast<void*>(uintptr_t{4096});
        return 0;
    }
    int counters(size_t n, unsigned** out) override {
        cnt = std::max(cnt, n);
        *out = reinterpret_cast<unsigned*>(uintptr_t{4096});
        return 0;
    }
    size_t ws = 0, cnt = 0;
};

class PoolScratch : public Scratch {
public:
    explicit PoolScratch(hipStream_t s) : s_(s) {}
    int workspace(size_t bytes, void** out) override {
        if (const int rc = take()) return rc;
        return mapped(lease_.workspace(bytes, out));
    }
    int counters(size_t n, unsigned** out) override {
        if (const int rc = take()) return rc;
        return mapped(lease_.counters(n, out));
    }

private:
    int take() {
        if (!have_) {
            int dev = 0;
            if (const int rc = device_of(s_, &dev)) return rc;
            lease_ = pool_of(dev)->lease(s_);
            have_ = true;
        }
        return mapped(lease_.status());
    }
    static int mapped(int rc) { return rc == Pool::kNeedsAlloc ? GEMM355_ERR_CAPTURE : rc; }
    hipStream_t s_;
    bool have_ = false;
    Pool::Lease lease_;
};

// ---------------------------------------------------------------------------
// Argument checks (BLAS xerbla numbering) and the dispatch of one call.
// ---------------------------------------------------------------------------
// Arguments are numbered as in gemm_f32: 1 M, 2 N, 3 K, 5 A, 6 lda, 7 B,
// 8 ldb, 10 C, 11 ldc (the _ex entry points add 2 and number transa, transb
// 1 and 2).  A is stored M x K (K x M when op(A) = A^T), B K x N (N x K).
int check_args(int trans, int64_t M, int64_t N, int64_t K, float alpha, const float* A,
               int64_t lda, const float* B, int64_t ldb, const float* C, int64_t ldc) {
    if (M < 0 || M > kMaxDim) return -1;
    if (N < 0 || N > kMaxDim) return -2;
    if (K < 0 || K > kMaxDim) return -3;
    const bool product = M > 0 && N > 0 && K > 0 && alpha != 0.f;
    const int64_t a_row = (trans & 1) ? M : K, b_row = (trans & 2) ? K : N;
    if (product && A == nullptr) return -5;
    if (lda < std::max<int64_t>(1, a_row)) return -6;
    if (product && B == nullptr) return -7;
    if (ldb < std::max<int64_t>(1, b_row)) return -8;
    if (M > 0 && N > 0 && C == nullptr) return -10;
    if (ldc < std::max<int64_t>(1, N)) return -11;
    return 0;
}

// The split-K configuration: slices of K chosen so that tiles x slices reaches
// kSplitKTarget workgroups, each slice at least kSplitKMinDepth deep (a
// multiple of BK), the partial tiles within kSplitKMaxBytes.  One slice runs
// the normal epilogue; more go through the workspace and the reduction.
int launch_splitk(const TileConfig& cfg, int trans, int64_t M, int64_t N, int64_t K, float alpha,
                  const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                  int64_t ldc, hipStream_t s, uint16_t* C16, Scratch& sc) {
    const int tiles_m = static_cast<int>((M + cfg.bm - 1) / cfg.bm);
    const int tiles_n = static_cast<int>((N + cfg.bn - 1) / cfg.bn);
    const int64_t tiles = int64_t{tiles_m} * tiles_n;
    int64_t slices = std::max<int64_t>(1, (kSplitKTarget + tiles - 1) / tiles);
    slices = std::min(slices, std::max<int64_t>(1, K / kSplitKMinDepth));
    slices = std::min(slices, std::max<int64_t>(1, kSplitKMaxBytes / (M * N * 4)));
    int64_t depth = round_up((K + slices - 1) / slices, cfg.bk);
    slices = (K + depth - 1) / depth;
    F32Args a{A, B, C, lda, ldb, ldc, static_cast<int>(M), static_cast<int>(N),
              static_cast<int>(K), alpha, beta, tiles_m, tiles_n};
    F32Variant v;
    v.vec = vec_ok(A, lda) && vec_ok(B, ldb);
    // every slice but the last is a whole number of BK-deep panels, and so is
    // the last one when K is
    v.masked = !v.vec || (M % cfg.bm) || (N % cfg.bn) || (K % cfg.bk);
    v.ta = (trans & 1) != 0;
    v.tb = (trans & 2) != 0;
    v.r16 = cfg.mode == GEMM355_MODE_F16R;
    if (log_debug() && !sc.dry())
        std::fprintf(stderr, "[gemm355] %s M=%lld N=%lld K=%lld %s path=split-K x%lld (k %lld)%s\n",
                     layout_name(cfg.mode, trans).c_str(), (long long)M, (long long)N,
                     (long long)K, format_config(cfg).c_str(), (long long)slices,
                     (long long)depth, v.masked ? " masked" : "");
    // binary16 output always goes through the reduction, which rounds
    if (slices == 1 && !C16) return sc.dry() ? 0 : status_of(launch_f32_splitk(a, v, s));
    void* ws = nullptr;
    if (const int rc = sc.workspace(static_cast<size_t>(slices * M * N) * 4, &ws)) return rc;
    if (sc.dry()) return 0;
    a.C = static_cast<float*>(ws);
    a.ldc = N;
    a.ksplit = static_cast<int>(depth);   // one slice too, when the output is binary16
    // the slices of a ragged split write partial tiles masked to M x N
    hipError_t e = launch_f32_splitk(a, v, s);
    if (e != hipSuccess) return status_of(e);
    if (C16)
        return status_of(launch_splitk_reduce16(static_cast<const float*>(ws),
                                                static_cast<int>(slices), static_cast<int>(M),
                                                static_cast<int>(N), alpha, beta, C16, ldc, s));
    return status_of(launch_splitk_reduce(static_cast<const float*>(ws), static_cast<int>(slices),
                                          static_cast<int>(M), static_cast<int>(N), alpha, beta,
                                          C, ldc, s));
}

// The few-rows configuration: slices of K so that column groups x row groups
// x slices reaches kRowsTarget workgroups, each slice a whole number of
// rows_depth_unit() (every wave at least one 64-deep chunk), the partial
// tiles within kSplitKMaxBytes.  Shapes whose B cannot be read 16 bytes at a
// time take the split-K configuration instead.  A call with few columns and
// more rows (N <= kRowsRows < M) runs as the transposed problem C^T =
// op(B)^T op(A)^T, whose few rows stream A, with C stored transposed: the
// few-columns form.
int launch_rows(const TileConfig& cfg, int trans, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                int64_t ldc, hipStream_t s, uint16_t* C16, Scratch& sc) {
    const bool ta_in = (trans & 1) != 0, tb_in = (trans & 2) != 0;
    const bool tc = N <= kRowsRows && M > kRowsRows;
    if (tc) {
        // C^T (N x M) = op(B)^T (N x K) op(A)^T (K x M): op(B)^T is B read
        // with the other layout flag, and likewise op(A)^T
        std::swap(M, N);
        std::swap(A, B);
        std::swap(lda, ldb);
    }
    const bool ta = tc ? !tb_in : ta_in, tb = tc ? !ta_in : tb_in;
    if (!rows_supported(ta, tb, B, lda, ldb, static_cast<int>(M), static_cast<int>(N),
                        static_cast<int>(K))) {
        if (tc) {
            std::swap(M, N);
            std::swap(A, B);
            std::swap(lda, ldb);
        }
        return launch_splitk(splitk_config(cfg.mode), trans, M, N, K, alpha, A, lda, B, ldb, beta,
                             C, ldc, s, C16, sc);
    }
    // Slice depth: two 64-deep chunks per wave (one pass of the kernel) when
    // that gives at least one workgroup per CU, one chunk when the grid would
    // be smaller; deeper slices when there would be more than kRowsMaxWgs
    // workgroups or the partial tiles would pass kSplitKMaxBytes.
    const int64_t unit = rows_depth_unit();
    const int64_t group = rows_group(static_cast<int>(M));
    const int64_t wgs = ((N + 63) / 64) * ((M + group - 1) / group);
    int64_t depth = 2 * unit;
    if (wgs * ((K + depth - 1) / depth) < kCUs) depth = unit;
    const int64_t max_slices = std::max<int64_t>(
        1, std::min(kRowsMaxWgs / wgs, kSplitKMaxBytes / std::max<int64_t>(1, M * round_up(N, 4) * 4)));
    if ((K + depth - 1) / depth > max_slices) depth = round_up((K + max_slices - 1) / max_slices, unit);
    const int64_t slices = (K + depth - 1) / depth;
    const bool r16 = cfg.mode == GEMM355_MODE_F16R;
    if (log_debug() && !sc.dry())
        std::fprintf(stderr, "[gemm355] %s M=%lld N=%lld K=%lld %s path=rows x%lld (k %lld)%s\n",
                     layout_name(cfg.mode, trans).c_str(), (long long)(tc ? N : M),
                     (long long)(tc ? M : N), (long long)K, format_config(cfg).c_str(),
                     (long long)slices, (long long)depth, C16 ? " f16-out" : "");
    const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
    float* P = nullptr;
    unsigned* counts = nullptr;
    if (slices > 1) {
        void* ws = nullptr;
        // partial rows are N rounded up to 4 floats apart
        int rc = sc.workspace(static_cast<size_t>(slices * M * round_up(N, 4)) * 4, &ws);
        if (rc == 0) rc = sc.counters(static_cast<size_t>(rows_counters(m, n)), &counts);
        if (rc) return rc;
        P = static_cast<float*>(ws);
    }
    if (sc.dry()) return 0;
    return status_of(launch_f32_rows(A, lda, ta, B, ldb, tb, r16, C, C16, ldc, tc, m, n, k, alpha,
                                     beta, static_cast<int>(depth), static_cast<int>(slices), P,
                                     counts, s));
}

// Whether a KS=3 call runs as its transposed problem with C stored
// transposed: the 16-row tile of the f32-panel ring, a C of at most 16
// columns and more rows, A stored M x K, and a transposed problem the ring
// takes (op(B)^T as A': 16-byte rows, and M' = N a multiple of 4 where it is
// stored K x N).
bool columns_form(const TileConfig& cfg, int trans, int64_t M, int64_t N, int64_t K,
                  const float* A, int64_t lda, const float* B, int64_t ldb) {
    const bool ta = (trans & 1) != 0, tb = (trans & 2) != 0;
    return cfg.ks == 3 && cfg.bk == 32 && cfg.bm == 16 && N <= kRowsRows && M > kRowsRows && !ta &&
           panel_ring_takes(!tb, true, B, ldb, A, lda, N, M, K);
}

// One KS=3 launch; tc: C stored transposed (the few-columns form).
int run_direct(const TileConfig& cfg_in, int trans, int64_t M, int64_t N, int64_t K, float alpha,
               const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
               int64_t ldc, hipStream_t s, uint16_t* C16, Scratch& sc, bool tc);

// The configurations that round the operands as they stage them (KS=3), on
// the grid of direct_grid.
int launch_direct(const TileConfig& cfg_in, int trans, int64_t M, int64_t N, int64_t K,
                  float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                  float beta, float* C, int64_t ldc, hipStream_t s, uint16_t* C16, Scratch& sc) {
    TileConfig cfg = cfg_in;
    // The 16-row tile of the f32-panel ring runs a C of at most 16 columns
    // and more rows as the transposed problem C^T = op(B)^T op(A)^T, whose few
    // rows stream A (stored M x K, so op(A)^T is the ring's B^T layout, read
    // in whole rows), with C stored transposed (the block-layout epilogue of
    // that layout writes C^T[row][col] to C[col * ldc + row]).
    if (columns_form(cfg, trans, M, N, K, A, lda, B, ldb)) {
        const bool tb_in = (trans & 2) != 0;
        return run_direct(cfg, (tb_in ? 0 : 1) | 2, N, M, K, alpha, B, ldb, A, lda, beta, C, ldc,
                          s, C16, sc, true);
    }
    return run_direct(cfg, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s, C16, sc, false);
}

int run_direct(const TileConfig& cfg_in, int trans, int64_t M, int64_t N, int64_t K, float alpha,
               const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
               int64_t ldc, hipStream_t s, uint16_t* C16, Scratch& sc, bool tc) {
    TileConfig cfg = cfg_in;
    const bool ta = (trans & 1) != 0, tb = (trans & 2) != 0;
    // the f32-panel ring (BK = 32) hands the shapes it does not take to the
    // register-staged kernel of the 64 x 64 tile (f16r) or to the split-K
    // tiles (f32)
    if (cfg.bk == 32 && !panel_ring_takes(ta, tb, A, lda, B, ldb, M, N, K)) {
        if (tc) return GEMM355_ERR_CONFIG;   // columns_form checked the transposed problem
        if (cfg.mode == GEMM355_MODE_F32)
            return launch_splitk(splitk_config(cfg.mode), trans, M, N, K, alpha, A, lda, B, ldb,
                                 beta, C, ldc, s, C16, sc);
        TileConfig fb;
        if (!parse_config(cfg.mode, "BM=64 BN=64 BK=64 KS=3", &fb)) return GEMM355_ERR_CONFIG;
        cfg = fb;
    }
    int n = 0;
    const DirectInstance* inst = nullptr;
    const DirectInstance* t = panel_ring_instances(cfg.mode, &n);
    for (int i = 0; i < n; ++i)
        if (t[i].cfg == cfg) inst = &t[i];
    if (cfg.mode == GEMM355_MODE_F16R) {
        t = direct_instances(&n);
        for (int i = 0; i < n; ++i)
            if (t[i].cfg == cfg) inst = &t[i];
    }
    if (!inst) return GEMM355_ERR_CONFIG;
    const DirectGrid dg = direct_grid(cfg, M, N, K);
    const int64_t tiles_m = dg.tiles_m, tiles_n = dg.tiles_n, tiles = tiles_m * tiles_n;
    const int64_t slices = dg.slices, depth = dg.depth;
    const int64_t tile_bytes = int64_t{cfg.bm} * cfg.bn * 4;
    const bool masked = !vec_ok(A, lda) || !vec_ok(B, ldb) || (M % cfg.bm) || (N % cfg.bn) ||
                        (K % cfg.bk);
    if (log_debug() && !sc.dry())
        std::fprintf(stderr, "[gemm355] %s M=%lld N=%lld K=%lld %s path=direct x%lld (k %lld)%s\n",
                     layout_name(cfg.mode, trans).c_str(), (long long)M, (long long)N,
                     (long long)K, format_config(cfg).c_str(), (long long)slices,
                     (long long)depth, masked ? " masked" : "");
    DirectArgs a{A, B, C, C16, nullptr, nullptr, lda, ldb, ldc, static_cast<int>(M),
                 static_cast<int>(N), static_cast<int>(K), alpha, beta,
                 static_cast<int>(tiles_m), static_cast<int>(tiles_n),
                 static_cast<int>(depth), static_cast<int>(slices), tc};
    if (slices > 1) {
        void* ws = nullptr;
        int rc = sc.workspace(static_cast<size_t>(slices * tiles * tile_bytes), &ws);
        if (rc == 0) rc = sc.counters(static_cast<size_t>(tiles), &a.counts);
        if (rc) return rc;
        a.P = static_cast<float*>(ws);
    }
    if (sc.dry()) return 0;
    return status_of(inst->launch(a, ta, tb, masked, s));
}

// whole_call: run the call as one piece (a part of a split call).
int launch_with(const TileConfig& cfg, int trans, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                int64_t ldc, hipStream_t s, uint16_t* C16, Scratch& sc, bool whole_call = false) {
    if (cfg.ks == 2)
        return launch_rows(cfg, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s, C16, sc);
    if (cfg.ks == 3)
        return launch_direct(cfg, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s, C16, sc);
    if (cfg.ks)
        return launch_splitk(cfg, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s, C16, sc);
    const RingBlock rb = whole_call ? RingBlock{M, N, K, 0.0}
                                    : ring_block(cfg, ring_rows(trans, A, lda, B, ldb), M, N, K);
    if (rb.mb < M || rb.nb < N || rb.kb < K) {
        // A ragged call of a ring configuration split as ring_block chose:
        // the ring runs the block (unmasked when it is whole tiles with
        // 16-byte aligned rows), the register-staged 64 x 64 tile adds the k
        // tail to the block (beta = 1), and the strips go to the
        // configurations of their shapes.
        TileConfig edge;
        if (!parse_config(cfg.mode, "BM=64 BN=64 BK=16 ST=2", &edge)) return GEMM355_ERR_CONFIG;
        int rc = launch_with(cfg, 0, rb.mb, rb.nb, rb.kb, alpha, A, lda, B, ldb, beta, C, ldc, s,
                             nullptr, sc, true);
        if (rc == 0 && rb.kb < K)
            rc = launch_with(edge, 0, rb.mb, rb.nb, K - rb.kb, alpha, A + rb.kb, lda,
                             B + rb.kb * ldb, ldb, 1.0f, C, ldc, s, nullptr, sc, true);
        if (rc == 0 && rb.nb < N)
            rc = launch_with(strip_config(cfg.mode, M, N - rb.nb), 0, M, N - rb.nb, K, alpha, A, lda,
                             B + rb.nb, ldb, beta, C + rb.nb, ldc, s, nullptr, sc, true);
        if (rc == 0 && rb.mb < M)
            rc = launch_with(strip_config(cfg.mode, M - rb.mb, rb.nb), 0, M - rb.mb, rb.nb, K, alpha,
                             A + rb.mb * lda, lda, B, ldb, beta, C + rb.mb * ldc, ldc, s, nullptr,
                             sc, true);
        return rc;
    }
    const int tiles_m = static_cast<int>((M + cfg.bm - 1) / cfg.bm);
    const int tiles_n = static_cast<int>((N + cfg.bn - 1) / cfg.bn);
    if (cfg.mode == GEMM355_MODE_F32) {
        int n = 0;
        const F32Instance* t = f32_instances(&n);
        for (int i = 0; i < n; ++i) {
            if (!(t[i].cfg == cfg)) continue;
            F32Args a{A, B, C, lda, ldb, ldc, static_cast<int>(M), static_cast<int>(N),
                      static_cast<int>(K), alpha, beta, tiles_m, tiles_n};
            F32Variant v;
            v.vec = vec_ok(A, lda) && vec_ok(B, ldb);
            v.ta = (trans & 1) != 0;
            v.tb = (trans & 2) != 0;
            v.masked = !v.vec || (M % cfg.bm) || (N % cfg.bn) || (K % cfg.bk);
            // a ring configuration deals its work to the CUs in equal runs
            // (stream-K) when whole rounds of tiles would leave CUs idle
            const RingSk sk =
                is_f32_ring(cfg) && f32_ring_takes(cfg, a, v) ? ring_sk(cfg, M, N, K) : RingSk{};
            if (sk.q > 0) {
                const int64_t tiles = int64_t{tiles_m} * tiles_n;
                a.sk_q = static_cast<int>(sk.q);
                a.sk_dp = static_cast<int>(sk.dp);
                a.sk_grid = static_cast<int>(sk.grid);
                void* ws = nullptr;
                int rc = sc.workspace(static_cast<size_t>(sk.grid * 2 * cfg.bm * cfg.bn) * 4, &ws);
                if (rc == 0) rc = sc.counters(static_cast<size_t>(tiles), &a.counts);
                if (rc) return rc;
                a.P = static_cast<float*>(ws);
            }
            if (sc.dry()) return 0;
            if (log_debug())
                std::fprintf(stderr, "[gemm355] %s M=%lld N=%lld K=%lld %s path=%s%s run %d\n",
                             layout_name(cfg.mode, trans).c_str(), (long long)M, (long long)N,
                             (long long)K, format_config(cfg).c_str(),
                             v.masked ? "masked" : "aligned", v.vec ? "" : " scalar-loads",
                             a.sk_q);
            return status_of(t[i].launch(a, v, s));
        }
        return GEMM355_ERR_CONFIG;
    }
    int n = 0;
    unsigned* counts = nullptr;
    const F16Instance* t = f16_instances(&n);
    for (int i = 0; i < n; ++i) {
        if (!(t[i].cfg == cfg)) continue;
        const int64_t mp = round_up(M, 256), np = round_up(N, 256), kp = round_up(K, 64);
        // a half-depth ring deals its work in equal runs (stream-K) when whole
        // rounds of tiles would leave slots idle; its partial tiles follow the
        // packed operands in the workspace
        const RingSk sk = is_f16_ring(cfg) ? ring_sk(cfg, M, N, K) : RingSk{};
        const int64_t q = sk.q;
        const int64_t packed_bytes = round_up((mp + np) * kp * 2, 256);
        void* ws = nullptr;
        int rc = sc.workspace(static_cast<size_t>(packed_bytes + sk.grid * 2 * cfg.bm * cfg.bn * 4),
                              &ws);
        if (rc == 0 && q > 0) rc = sc.counters(static_cast<size_t>(tiles_m) * tiles_n, &counts);
        if (rc) return rc;
        if (sc.dry()) return 0;
        uint16_t* A16 = static_cast<uint16_t*>(ws);
        uint16_t* B16t = A16 + mp * kp;
        hipError_t e = launch_pack(A, lda, (trans & 1) != 0, B, ldb, (trans & 2) != 0, static_cast<int>(M),
                        static_cast<int>(N), static_cast<int>(K), A16, B16t, mp, np, kp, cfg.bk,
                        s);
        if (e != hipSuccess) return status_of(e);
        F16Args a{A16, B16t, C, kp / cfg.bk, ldc, static_cast<int>(M), static_cast<int>(N), alpha,
                  beta, tiles_m, tiles_n};
        a.C16 = C16;
        if (q > 0) {
            a.sk_q = static_cast<int>(q);
            a.sk_dp = static_cast<int>(sk.dp);
            a.sk_grid = static_cast<int>(sk.grid);
            a.P = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + packed_bytes);
            a.counts = counts;
        }
        if (log_debug())
            std::fprintf(stderr, "[gemm355] %s M=%lld N=%lld K=%lld %s path=%s%s run %lld\n",
                         layout_name(cfg.mode, trans).c_str(), (long long)M, (long long)N,
                         (long long)K, format_config(cfg).c_str(),
                         ((M % cfg.bm) || (N % cfg.bn)) ? "masked-store" : "aligned",
                         C16 ? " f16-out" : "", (long long)q);
        return status_of(t[i].launch(a, s));
    }
    return GEMM355_ERR_CONFIG;
}

// C16 != NULL: the f16-output variant (f16r mode only): C is stored as
// binary16 in C16 and the f32 result is rounded to nearest even; C is unused.
// sc: where the call's scratch comes from (NULL: a lease of the device's pool).
int gemm(int mode, int trans, int64_t M, int64_t N, int64_t K, float alpha, const float* A,
         int64_t lda, const float* B, int64_t ldb, float beta, float* C, int64_t ldc, void* stream,
         const TileConfig* force, uint16_t* C16, Scratch* sc = nullptr) {
    const float* c_arg = C16 ? reinterpret_cast<const float*>(C16) : C;
    const int bad = check_args(trans, M, N, K, alpha, A, lda, B, ldb, c_arg, ldc);
    if (bad) return bad;
    if (C16 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    if (M == 0 || N == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0 || alpha == 0.f) {
        if (log_debug())
            std::fprintf(stderr, "[gemm355] %s M=%lld N=%lld K=%lld path=beta-only%s\n",
                         mode_name(mode), (long long)M, (long long)N, (long long)K,
                         C16 ? " f16-out" : "");
        if (C16)
            return status_of(
                launch_scale_c16(C16, ldc, static_cast<int>(M), static_cast<int>(N), beta, s));
        return status_of(launch_scale_c(C, ldc, static_cast<int>(M), static_cast<int>(N), beta, s));
    }
    TileConfig cfg;
    if (force) {
        cfg = *force;
    } else {
        Source src;
        const int rc = select_config(mode, trans, M, N, K, A, lda, B, ldb, beta, &cfg, &src);
        if (rc) return rc;
    }
    // plan (nothing launched), take the scratch the plan needs, then launch:
    // a failure to obtain scratch leaves C untouched
    DryScratch plan;
    int rc = launch_with(cfg, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s, C16, plan);
    if (rc) return rc;
    PoolScratch pooled(s);
    Scratch& use = sc ? *sc : pooled;
    if (plan.ws || plan.cnt) {
        rc = use.reserve(plan.ws, plan.cnt);
        if (rc) return rc;
    }
    return launch_with(cfg, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, s, C16, use);
}

// ---------------------------------------------------------------------------
// Tuning cache file: one entry per line,
//   <mode> <M> <N> <K> <vec_a> <vec_b> <beta0> BM=.. BN=.. BK=.. WM=.. WN=.. GM=..
// ---------------------------------------------------------------------------
size_t load_cache_locked(State& st, const char* path) {
    FILE* f = std::fopen(path, "r");
    if (!f) return 0;
    char line[512];
    size_t n = 0;
    while (std::fgets(line, sizeof line, f)) {
        char mode_s[16];
        long long M, N, K;
        int va, vb, b0, off = 0;
        if (std::sscanf(line, "%15s %lld %lld %lld %d %d %d %n", mode_s, &M, &N, &K, &va, &vb,
                        &b0, &off) != 7)
            continue;
        int mode = -1, trans = -1;
        for (int m = 0; m < 2 && mode < 0; ++m)
            for (int t = 0; t < 4; ++t)
                if (layout_name(m, t) == mode_s) {
                    mode = m;
                    trans = t;
                    break;
                }
        if (mode < 0 || M < 0 || N < 0 || K < 0) continue;
        std::string rest(line + off);
        while (!rest.empty() && (rest.back() == '\n' || rest.back() == '\r')) rest.pop_back();
        TileConfig c;
        if (!parse_config(mode, rest.c_str(), &c)) continue;
        st.cache[Key{mode, M, N, K, va != 0, vb != 0, b0 != 0, trans}] = c;
        ++n;
    }
    std::fclose(f);
    return n;
}

int save_cache_locked(State& st, const char* path) {
    if (!path || !*path) return GEMM355_ERR_BUFFER;
    const std::string tmp = std::string(path) + ".tmp";
    FILE* f = std::fopen(tmp.c_str(), "w");
    if (!f) return GEMM355_ERR_BUFFER;
    int n = 0;
    for (const auto& kv : st.cache) {
        const Key& k = kv.first;
        std::fprintf(f, "%s %lld %lld %lld %d %d %d %s\n", layout_name(k.mode, k.trans).c_str(),
                     (long long)k.M,
                     (long long)k.N, (long long)k.K, k.vec_a, k.vec_b, k.beta0,
                     format_config(kv.second).c_str());
        ++n;
    }
    std::fclose(f);
    if (std::rename(tmp.c_str(), path) != 0) return GEMM355_ERR_BUFFER;
    return n;
}

// ---------------------------------------------------------------------------
// The autotuner (phobos docs, "gemm, f32", section "Tuning"): stage 1 times
// every compiled configuration a few times and drops those that fail; stage 2
// re-times the fastest few over shuffled rounds, one sample of each per round,
// so the finalists see the same clocks (the lab's sweep() helper).  A sample
// of a short call is several back-to-back calls between two events (as many
// as fill kTuneSampleMs, at most kTuneMaxReps), per call: the time of a call
// in a stream of calls, which a single call would overstate by the host's
// launch work (a few microseconds, more for calls of several launches) when
// that is not hidden behind the previous call.
// ---------------------------------------------------------------------------
constexpr float kTuneSampleMs = 0.2f;
constexpr int kTuneMaxReps = 16;

struct Timed {
    TileConfig cfg;
    int reps = 1;
    std::vector<float> ms;
    float median() const {
        std::vector<float> v = ms;
        std::sort(v.begin(), v.end());
        return v.empty() ? 1e30f : v[v.size() / 2];
    }
};

// One sample: `reps` calls of `cfg` between two events; *ms = time per call.
int time_once(const TileConfig& cfg, int trans, int64_t M, int64_t N, int64_t K, const float* A,
              int64_t lda, const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
              hipStream_t s, hipEvent_t e0, hipEvent_t e1, int reps, float* ms) {
    hipError_t e = hipEventRecord(e0, s);
    if (e != hipSuccess) return status_of(e);
    for (int i = 0; i < reps; ++i) {
        const int rc = gemm(cfg.mode, trans, M, N, K, 1.0f, A, lda, B, ldb, beta, C, ldc, s, &cfg,
                            nullptr);
        if (rc) return rc;
    }
    e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
    *ms /= static_cast<float>(reps);
    return status_of(e);
}

int tune(int mode, int trans, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
         const float* B, int64_t ldb, float beta, int64_t ldc, void* stream) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    float* C = nullptr;
    // a stand-in C pointer for the argument check; the real scratch comes next
    const int bad = check_args(trans, M, N, K, 1.0f, A, lda, B, ldb,
                               reinterpret_cast<const float*>(uintptr_t{16}), ldc);
    if (bad) return bad;
    if (M == 0 || N == 0 || K == 0) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMalloc(&C, static_cast<size_t>(M) * ldc * sizeof(float));
    if (e != hipSuccess) return GEMM355_ERR_ALLOC;
    e = hipMemsetAsync(C, 0, static_cast<size_t>(M) * ldc * sizeof(float), s);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    int rc = status_of(e);
    std::vector<Timed> ok;
    if (rc == 0) {
        for (const TileConfig& cfg : configs_of(mode)) {
            Timed t{cfg, 1, {}};
            float ms = 0.f;
            // warm-up, then the sample size from a second single call
            int r = time_once(cfg, trans, M, N, K, A, lda, B, ldb, beta, C, ldc, s, e0, e1, 1, &ms);
            if (r == 0) r = time_once(cfg, trans, M, N, K, A, lda, B, ldb, beta, C, ldc, s, e0, e1, 1, &ms);
            if (r == 0 && ms > 0.f && ms < kTuneSampleMs)
                t.reps = std::min(kTuneMaxReps, static_cast<int>(std::ceil(kTuneSampleMs / ms)));
            for (int i = 0; i < 3 && r == 0; ++i) {
                r = time_once(cfg, trans, M, N, K, A, lda, B, ldb, beta, C, ldc, s, e0, e1, t.reps, &ms);
                if (r == 0) t.ms.push_back(ms);
            }
            if (r != 0) {
                (void)hipGetLastError();   // a failing candidate is skipped
                if (log_debug())
                    std::fprintf(stderr, "[gemm355] tune: %s failed (%d), skipped\n",
                                 format_config(cfg).c_str(), r);
                continue;
            }
            ok.push_back(t);
        }
        std::sort(ok.begin(), ok.end(),
                  [](const Timed& a, const Timed& b) { return a.median() < b.median(); });
        if (ok.size() > 4) ok.resize(4);
        for (Timed& t : ok) t.ms.clear();
        uint64_t lcg = 0x9E3779B97F4A7C15ull;
        std::vector<size_t> order(ok.size());
        for (int round = 0; round < 12 && !ok.empty(); ++round) {
            for (size_t i = 0; i < order.size(); ++i) order[i] = i;
            for (size_t i = order.size(); i > 1; --i) {   // Fisher-Yates with an LCG
                lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
                std::swap(order[i - 1], order[(lcg >> 33) % i]);
            }
            for (size_t i : order) {
                float ms = 0.f;
                if (time_once(ok[i].cfg, trans, M, N, K, A, lda, B, ldb, beta, C, ldc, s, e0, e1,
                              ok[i].reps, &ms) == 0)
                    ok[i].ms.push_back(ms);
            }
        }
        if (ok.empty()) {
            rc = GEMM355_ERR_CONFIG;
        } else {
            const Timed* best = &ok[0];
            for (const Timed& t : ok)
                if (t.median() < best->median()) best = &t;
            if (log_debug())
                for (const Timed& t : ok)
                    std::fprintf(stderr, "[gemm355] tune %s M=%lld N=%lld K=%lld %s: %.4f ms%s\n",
                                 layout_name(mode, trans).c_str(), (long long)M, (long long)N, (long long)K,
                                 format_config(t.cfg).c_str(), t.median(),
                                 &t == best ? "  <- chosen" : "");
            State& st = state();
            std::lock_guard<std::mutex> lock(st.mu);
            read_env_locked(st);
            st.cache[Key{mode, M, N, K, vec_ok(A, lda), vec_ok(B, ldb), beta == 0.f, trans}] =
                best->cfg;
            if (!st.cache_path.empty()) save_cache_locked(st, st.cache_path.c_str());
        }
    }
    (void)hipStreamSynchronize(s);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipFree(C);
    return rc;
}

int copy_out(const std::string& s, char* buf, size_t len) {
    if (!buf || len == 0) return GEMM355_ERR_BUFFER;
    if (s.size() + 1 > len) {
        std::memcpy(buf, s.data(), len - 1);
        buf[len - 1] = '\0';
        return GEMM355_ERR_BUFFER;
    }
    std::memcpy(buf, s.c_str(), s.size() + 1);
    return 0;
}

}  // namespace
}  // namespace g355

using namespace g355;

extern "C" {

int gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
             const float* B, int64_t ldb, float beta, float* C, int64_t ldc, void* stream) {
    return gemm(GEMM355_MODE_F32, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                nullptr, nullptr);
}

int gemm_f16r_f32acc(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
                     const float* B, int64_t ldb, float beta, float* C, int64_t ldc,
                     void* stream) {
    return gemm(GEMM355_MODE_F16R, 0, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                nullptr, nullptr);
}

}  // extern "C"

namespace {

// The _ex entry points: transa, transb must be 0 or 1 (codes -1, -2); the
// other argument codes move up by two (BLAS sgemm numbering).
int trans_of(int transa, int transb, int* trans) {
    if (transa != 0 && transa != 1) return -1;
    if (transb != 0 && transb != 1) return -2;
    *trans = transa | (transb << 1);
    return 0;
}
int shift_ex(int rc) { return rc < 0 && rc > -100 ? rc - 2 : rc; }

}  // namespace

extern "C" {

int gemm_f32_ex(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                int64_t ldc, void* stream) {
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    return shift_ex(gemm(GEMM355_MODE_F32, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream, nullptr, nullptr));
}

int gemm_f16r_f32acc_ex(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                        const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                        float* C, int64_t ldc, void* stream) {
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    return shift_ex(gemm(GEMM355_MODE_F16R, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                         stream, nullptr, nullptr));
}

int gemm_f16r_f16out(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                     const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                     uint16_t* C16, int64_t ldc, void* stream) {
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    return shift_ex(gemm(GEMM355_MODE_F16R, trans, M, N, K, alpha, A, lda, B, ldb, beta, nullptr,
                         ldc, stream, nullptr, C16));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The entry point that allocates nothing (gemm355_gemm_noalloc): its scratch
// is this file-scope device array, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// names a stand-in, not device memory): the first call on a device looks up
// the device address of that GPU's copy once, and every launch takes that.
// Layout: kFixedCounters arrival counters, then the workspace.
// ---------------------------------------------------------------------------
namespace g355 {
namespace {
constexpr size_t kFixedScratchBytes = size_t{160} << 20;
constexpr size_t kFixedCounters = 16384;
constexpr size_t kFixedCounterBytes = kFixedCounters * sizeof(unsigned);   // 64 KiB
}  // namespace
}  // namespace g355

static __device__ __align__(256) unsigned char scratch[g355::kFixedScratchBytes];

namespace g355 {
namespace {

// The device address of the copy of `scratch` on the device of stream s,
// looked up once per device with that device current (the caller's current
// device is restored).
int fixed_scratch_base(hipStream_t s, unsigned char** out) {
    int dev = 0;
    if (const int rc = device_of(s, &dev)) return rc;
    static std::mutex mu;
    static std::map<int, unsigned char*> base;
    std::lock_guard<std::mutex> lock(mu);
    auto it = base.find(dev);
    if (it == base.end()) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
        void* ptr = nullptr;
        if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess) return status_of(e);
        if (!ptr) return GEMM355_ERR_INTERNAL;
        it = base.emplace(dev, static_cast<unsigned char*>(ptr)).first;
    }
    *out = it->second;
    return 0;
}

class FixedScratch : public Scratch {
public:
    FixedScratch(unsigned char* base, hipStream_t s) : base_(base), s_(s) {}
    int workspace(size_t bytes, void** out) override {
        if (bytes > kFixedScratchBytes - kFixedCounterBytes) return GEMM355_ERR_SCRATCH;
        *out = base_ + kFixedCounterBytes;
        return 0;
    }
    int counters(size_t n, unsigned** out) override {
        if (n > kFixedCounters) return GEMM355_ERR_SCRATCH;
        *out = reinterpret_cast<unsigned*>(base_);
        return 0;
    }
    // the array keeps the last call's contents: the counters this call uses
    // are cleared (by a kernel on the call's stream) before its launches
    int reserve(size_t bytes, size_t n) override {
        if (bytes > kFixedScratchBytes - kFixedCounterBytes || n > kFixedCounters)
            return GEMM355_ERR_SCRATCH;
        if (n == 0) return 0;
        return status_of(launch_fill_u32(reinterpret_cast<unsigned*>(base_),
                                         static_cast<int64_t>(n), 0u, s_));
    }

private:
    unsigned char* base_;
    hipStream_t s_;
};

}  // namespace
}  // namespace g355

extern "C" {

int gemm355_gemm_noalloc(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                         float beta, float* C, int64_t ldc, void* stream) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    unsigned char* base = nullptr;
    if (const int rc = fixed_scratch_base(static_cast<hipStream_t>(stream), &base)) return rc;
    FixedScratch fixed(base, static_cast<hipStream_t>(stream));
    return shift_ex(gemm(mode, trans, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                         nullptr, nullptr, &fixed));
}

int gemm355_tune(int mode, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                 const float* B, int64_t ldb, float beta, int64_t ldc, void* stream) {
    return tune(mode, 0, M, N, K, A, lda, B, ldb, beta, ldc, stream);
}

int gemm355_tune_ex(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                    const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                    int64_t ldc, void* stream) {
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    return shift_ex(tune(mode, trans, M, N, K, A, lda, B, ldb, beta, ldc, stream));
}

int gemm355_get_config_ex(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                          int64_t lda, int64_t ldb, int64_t ldc, float beta, char* buf,
                          size_t len) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    const float* aligned = reinterpret_cast<const float*>(uintptr_t{256});
    const int bad = check_args(trans, M, N, K, 1.0f, aligned, lda, aligned, ldb, aligned, ldc);
    if (bad) return shift_ex(bad);
    TileConfig cfg;
    Source src;
    const int rc =
        select_config(mode, trans, M, N, K, aligned, lda, aligned, ldb, beta, &cfg, &src);
    if (rc) return rc;
    const char* sname = src == Source::Pin ? "pin" : src == Source::Tuned ? "tuned" : "heuristic";
    return copy_out(format_config(cfg) + " source=" + sname, buf, len);
}

int gemm355_get_plan_ex(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, float beta, char* buf, size_t len) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    int trans = 0;
    if (const int bad = trans_of(transa, transb, &trans)) return bad;
    const float* aligned = reinterpret_cast<const float*>(uintptr_t{256});
    const int bad = check_args(trans, M, N, K, 1.0f, aligned, lda, aligned, ldb, aligned, ldc);
    if (bad) return shift_ex(bad);
    TileConfig cfg;
    Source src;
    const int rc =
        select_config(mode, trans, M, N, K, aligned, lda, aligned, ldb, beta, &cfg, &src);
    if (rc) return rc;
    const RingRows rows = ring_rows(trans, aligned, lda, aligned, ldb);
    const RingBlock b = ring_block(cfg, rows, M, N, K);
    const bool vec = vec_ok(aligned, lda) && vec_ok(aligned, ldb);
    std::string form;
    if (cfg.ks == 1) form = "split-k";
    else if (cfg.ks == 2) form = N <= kRowsRows && M > kRowsRows ? "columns" : "rows";
    else if (cfg.ks == 3)
        form = std::string(mode == GEMM355_MODE_F16R ? "round-on-load" : "panel-ring") +
               (columns_form(cfg, trans, M, N, K, aligned, lda, aligned, ldb) ? "-columns" : "");
    else if (mode == GEMM355_MODE_F16R) form = (b.mb % cfg.bm || b.nb % cfg.bn) ? "packed-masked" : "packed";
    else if (is_f32_ring(cfg) && !rows.none())
        form = rows.aligned() && b.mb % cfg.bm == 0 && b.nb % cfg.bn == 0 && b.kb % 16 == 0
                   ? "ring" : "ring-masked";
    else form = (!vec || M % cfg.bm || N % cfg.bn || K % cfg.bk) ? "tiles-masked" : "tiles";
    const std::string out = "form=" + form + " block=" + std::to_string(b.mb) + "x" +
                            std::to_string(b.nb) + "x" + std::to_string(b.kb) +
                            (vec ? "" : " rows=4-byte");
    return copy_out(out, buf, len);
}

int gemm355_get_config(int mode, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                       int64_t ldc, float beta, char* buf, size_t len) {
    const int rc = gemm355_get_config_ex(mode, 0, 0, M, N, K, lda, ldb, ldc, beta, buf, len);
    return rc < 0 && rc > -100 ? rc + 2 : rc;
}

int gemm355_set_config(int mode, const char* spec) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    State& st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    read_env_locked(st);
    if (!spec || !*spec) {
        st.pin_set[mode] = false;
        st.pin_bad[mode] = false;
        return 0;
    }
    TileConfig c;
    if (!parse_config(mode, spec, &c)) return GEMM355_ERR_CONFIG;
    st.pin[mode] = c;
    st.pin_set[mode] = true;
    st.pin_bad[mode] = false;
    return 0;
}

int gemm355_parse_config(int mode, const char* spec, char* buf, size_t len) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    TileConfig c;
    if (!spec || !parse_config(mode, spec, &c)) return GEMM355_ERR_CONFIG;
    return copy_out(format_config(c), buf, len);
}

int gemm355_list_configs(int mode, char* buf, size_t len) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    std::string all;
    const std::vector<TileConfig> cs = configs_of(mode);
    for (const TileConfig& c : cs) all += format_config(c) + "\n";
    const int rc = copy_out(all, buf, len);
    return rc ? rc : static_cast<int>(cs.size());
}

int gemm355_cache_load(const char* path) {
    State& st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    read_env_locked(st);
    if (!path || !*path) return GEMM355_ERR_BUFFER;
    st.cache_path = path;
    return static_cast<int>(load_cache_locked(st, path));
}

int gemm355_cache_save(const char* path) {
    State& st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    read_env_locked(st);
    if (path && *path) st.cache_path = path;
    return save_cache_locked(st, st.cache_path.c_str());
}

void gemm355_cache_clear(void) {
    State& st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    read_env_locked(st);
    st.cache.clear();
}

const char* gemm355_strerror(int status) {
    switch (status) {
        case 0: return "success";
        case -1: return "invalid argument 1 (M)";
        case -2: return "invalid argument 2 (N)";
        case -3: return "invalid argument 3 (K)";
        case -5: return "invalid argument 5 (A is NULL)";
        case -6: return "invalid argument 6 (lda < max(1, K))";
        case -7: return "invalid argument 7 (B is NULL)";
        case -8: return "invalid argument 8 (ldb < max(1, N))";
        case -10: return "invalid argument 10 (C is NULL)";
        case -11: return "invalid argument 11 (ldc < max(1, N))";
        case GEMM355_ERR_CONFIG: return "tile configuration unknown or not compiled";
        case GEMM355_ERR_ALLOC: return "device allocation failed";
        case GEMM355_ERR_MODE: return "unknown mode";
        case GEMM355_ERR_BUFFER: return "output buffer too small or file error";
        case GEMM355_ERR_INTERNAL: return "internal error";
        case GEMM355_ERR_CAPTURE:
            return "the call needs device scratch that is not allocated yet, and the stream is "
                   "being captured (run the call once before capturing, or use "
                   "gemm355_gemm_noalloc)";
        case GEMM355_ERR_SCRATCH:
            return "the call needs more scratch than the fixed array of gemm355_gemm_noalloc holds";
        default: break;
    }
    if (status > 0) return hipGetErrorString(static_cast<hipError_t>(status));
    return "unknown status";
}

const char* gemm355_version(void) { return "0.1.0"; }

int gemm355_roof_mfma(int mode, int form, int64_t iters, int blocks, float* sink,
                      double* flops_out, void* stream) {
    if (mode != GEMM355_MODE_F32 && mode != GEMM355_MODE_F16R) return GEMM355_ERR_MODE;
    if ((form != 0 && form != 1) || iters < 1 || blocks < 1 || !sink || !flops_out)
        return GEMM355_ERR_BUFFER;
    return status_of(launch_roof_mfma(mode, form, iters, blocks, sink, flops_out,
                                      static_cast<hipStream_t>(stream)));
}

int gemm355_roof_fma(int64_t iters, int blocks, float* sink, double* flops_out, void* stream) {
    if (iters < 1 || blocks < 1 || !sink || !flops_out) return GEMM355_ERR_BUFFER;
    return status_of(launch_roof_fma(iters, blocks, sink, flops_out, static_cast<hipStream_t>(stream)));
}

int gemm355_roof_hbm(const void* buf, int64_t bytes, int blocks, float* sink, void* stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 || blocks < 1 ||
        (reinterpret_cast<uintptr_t>(buf) & 15))
        return GEMM355_ERR_BUFFER;
    return status_of(launch_roof_hbm(buf, bytes, blocks, sink, static_cast<hipStream_t>(stream)));
}

int gemm355_copy_f32(const float* src, float* dst, int64_t n, void* stream) {
    if (n < 0 || ((!src || !dst) && n > 0)) return GEMM355_ERR_BUFFER;
    if (n == 0) return 0;
    if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return GEMM355_ERR_BUFFER;
    return status_of(launch_copy_f32(src, dst, n, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
