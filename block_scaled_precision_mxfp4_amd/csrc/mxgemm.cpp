// libmxgemm host library: argument validation, kernel/tile/split planning,
// split-K workspace management and the C-ABI entry points of libmxgemm.h.
//
// Planning follows the idea of the asm_f4gemm README's "Tile selection
// heuristic" (count how many rounds of workgroups the compute units need
// for each tile shape and prefer fewer, larger-tile rounds, iterating
// candidates in a fixed order so the choice is reproducible), extended with
// a per-tile cost so that tiles of different sizes and the split-K
// reduction can be compared, and with the skinny streaming kernels for
// M <= 16 (waves split K) and 16 < M <= 64 (waves split the rows of B and
// share A through LDS).
#include "libmxgemm.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "mx_args.hpp"

namespace mx {
// GEMV (mx_gemv.hip): M == 1 with A in format a_fmt (0 FP4, 1..4 FP8 E4M3,
// BF8 E5M2, FP6 E2M3, FP6 E3M2), or 2 <= M <= 8 with FP4 A; row-major B,
// K % 2048 == 0, 16-byte aligned scale rows, split 1; one workgroup per 4
// rows of B.
void launch_gemv(int a_fmt, const GemmArgs &g, int grid, hipStream_t s);
}  // namespace mx

namespace {

using mx::GemmArgs;

constexpr int kMaxK = 1 << 24;
static_assert(MXGEMM_NOALLOC_SCRATCH_BYTES == mx::kScratchBytes, "header and library agree on the scratch size");
constexpr int kMaxDevices = 64;
constexpr int kSplits[] = {1, 2, 4, 8, 16};

struct Plan {
    int family = 0;  // 0 tiled, 1 skinny (M <= 16), 2 skinny rows (16 < M <= 64), 3 tiled with
                     // a wider A, 4 GEMV (M <= 8)
    int index = 0;   // index into the kernel table of the family
    int bm = 0, bn = 0;
    int split = 1;
    int kb_per_split = 0;
    int tiles_m = 0, tiles_n = 0;
    int64_t grid = 0;
    bool lean = false;  // rows kernel: the two-slot ring (two workgroups per CU)
    size_t counter_bytes = 0;
    size_t ws_bytes = 0;
    const char *name = "";
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int cdiv(int a, int b) { return (a + b - 1) / b; }

// Split s over KB scale blocks in chunks of whole `gran`-block units (the
// tiled kernel's 256-K stage: 8 blocks; the skinny kernel's 4-step scale
// group: 16 blocks); returns blocks per chunk and the number of non-empty
// chunks.
std::pair<int, int> split_chunks(int KB, int s, int gran)
{
    int per = cdiv(cdiv(KB, s), gran) * gran;
    return {per, cdiv(KB, per)};
}

// Cost model of the tiled kernel: a measured time per 256-K stage for one
// round of workgroups of each tile (its occupancy's workgroups per CU at
// once), scaled down to 0.5 + 0.5 * the filled fraction when a single round
// leaves slots idle; times the rounds and stages; plus, for split K, 1 us per
// chunk, the partials' round trip at 5 TB/s and the last workgroup's reads.
// Fitted on MI355X to a sweep of every tile at splits 1, 2, 4, 8 over 15
// shapes (128x256x512 ... 8192x8192x2048, 2048x2048x8192, 1024x4096x16384,
// 4352^2 x 4096): it picks the measured best on all of them.  The times only
// rank candidates; the bench reports measured numbers.
double tile_stage_seconds(int bm, int bn)
{
    if (bm == 256 && bn == 256)
        return 1.6e-6;
    if (bm == 256)
        return 1.4e-6;
    if (bm == 128)
        return 1.2e-6;
    return 1.0e-6;
}
constexpr double kTileChunkCost = 1e-6;
constexpr double kHbm = 5.0e12;
// the 8-bit tiles' model: matrix time at 40 % of a CU's peak against the
// operand loads at 65 GB/s per CU, 2 us per split chunk (fitted before the
// split fix-up batched its loads)
constexpr double kCuFlops = 4.0 * 4096.0 * 2.4e9;
constexpr double kMatrixFraction = 0.4;
constexpr double kCuLoadRate = 65e9;
constexpr double kSplitChunkCost = 2e-6;
// The skinny kernels split K only into chunks of at least 64 scale blocks
// (2048 K): a sweep of splits 1..16 over 20 shapes with M <= 64 on MI355X
// found every shorter chunk slower than the next smaller split (the
// partial-sum tail outweighs the extra parallelism).
constexpr int kMinSkinnyChunk = 64;
constexpr double kCuL2 = 64.0 * 2.4e9;

// The GEMV (mx_gemv.hip) takes M == 1 (A in any format) and 2 <= M <= 8
// (FP4 A) with a row-major B when K is a multiple of its 2048-K chunk and
// its 4-row workgroups fill at least one per CU (N >= 4 * CUs); unsplit.
// MXGEMM_GEMV=0 keeps such shapes on the skinny kernel.
bool gemv_applies(int M, int N, int K, int b_packed, int split_req, int num_cu, int a_format)
{
    if (M < 1 || M > 8 || (M > 1 && a_format != MXGEMM_FMT_FP4) || b_packed || K % 2048 || split_req > 1 ||
        (int64_t)cdiv(N, 4) < num_cu)
        return false;
    const char *e = std::getenv("MXGEMM_GEMV");
    return !(e && std::strcmp(e, "0") == 0) && !std::getenv("MXGEMM_FORCE_NR");
}

Plan plan_for(int M, int N, int K, int b_packed, int split_req, int num_cu, bool tiled_only = false,
              int force_nr = 0, int a_format = MXGEMM_FMT_FP4, bool allow_gemv = true)
{
    const int KB = K / 32;
    if (num_cu <= 0)
        num_cu = 256;
    Plan best;
    double best_t = 1e300;

    auto consider_split = [&](int s) { return split_req <= 0 || s == split_req; };

    int n_tile = 0, n_skinny = 0, n_rows = 0;  // table sizes (the planner indexes them directly)
    const mx::TileKernel *tile = mx::tile_kernels(&n_tile);
    const mx::SkinnyKernel *skinny = mx::skinny_kernels(&n_skinny);
    const mx::RowsKernel *rows = mx::rows_kernels(&n_rows);
    if (M > 16 && M <= 64 && !tiled_only) {
        // Rows kernel: the four waves of a workgroup own 4 x 16 rows of B
        // and share one K chunk, with A staged once per workgroup.  The split
        // is the smallest that gives most CUs a workgroup while every chunk
        // keeps at least two batches (measured on MI355X: 64x7168x16384
        // fastest at split 2; split 4 moves the data faster with two
        // workgroups per CU but its partial-sum tail costs more than that).
        const int mg = cdiv(M, 16);
        const int idx = mg - 2;
        const int rows_wg = 64 * rows[idx].nrw;
        const int tiles = cdiv(N, rows_wg);
        int chosen = -1;
        for (int s : kSplits) {
            if (!consider_split(s))
                continue;
            auto [per, eff] = split_chunks(KB, s, 16);
            if (split_req <= 0) {
                if (s > 1 && (eff < s || per < kMinSkinnyChunk))
                    break;
                chosen = s;
                if ((int64_t)tiles * eff * 5 >= 4LL * num_cu)
                    break;
            } else {
                chosen = s;
            }
        }
        if (chosen < 0)
            chosen = 1;
        auto [per, eff] = split_chunks(KB, chosen, 16);
        best.family = 2;
        best.index = idx;
        best.bm = mg * 16;
        best.bn = rows_wg;
        best.split = eff;
        best.kb_per_split = per;
        best.tiles_m = 1;
        best.tiles_n = tiles;
        best.grid = (int64_t)tiles * eff;
        best.name = rows[idx].name[a_format];
        // more workgroups than CUs: with FP4 A and row-major B the four-slot
        // ring's 132 KiB of LDS leaves one workgroup per CU, the two-slot
        // ring fits two (64x28672x8192, 448 workgroups: 37.4 -> 34.1 us on
        // MI355X; at or below one workgroup per CU the deeper ring is faster)
        if (a_format == MXGEMM_FMT_FP4 && !b_packed && best.grid > num_cu) {
            best.lean = true;
            best.name = rows[idx].lean_name;
        }
        const size_t part = (size_t)rows_wg * mg * 16 * 4;
        best.counter_bytes = best.split > 1 ? (size_t)tiles * 4 : 0;
        best.ws_bytes = best.split > 1 ? (size_t)tiles * best.split * part : 0;
        return best;
    }
    if (!tiled_only && allow_gemv && force_nr <= 1 &&
        gemv_applies(M, N, K, b_packed, split_req, num_cu > 0 ? num_cu : 256, a_format)) {
        best.family = 4;
        best.bm = M;
        best.bn = 4;
        best.split = 1;
        best.kb_per_split = KB;
        best.tiles_m = 1;
        best.tiles_n = cdiv(N, 4);
        best.grid = best.tiles_n;
        best.name = M == 1 ? "gemv_m1_n4" : M <= 4 ? "gemv_m4_n4" : "gemv_m8_n4";
        return best;
    }
    if (M <= 16 && !tiled_only) {
        // Skinny kernel: a workgroup owns 16*nr rows of B and one K chunk.
        // Splitting K costs every split workgroup a serialized tail (partial
        // write-back, counter, read-back), so the split is the smallest that
        // gives most CUs a workgroup (measured on MI355X: 1x8192x8192
        // fastest with nr 1, unsplit).
        int nr = 1;
        if (const char *e = std::getenv("MXGEMM_FORCE_NR"))
            nr = std::atoi(e) >= 4 ? 4 : (std::atoi(e) >= 2 ? 2 : 1);
        if (force_nr > 0)
            nr = force_nr;
        const int nri = nr == 1 ? 0 : (nr == 2 ? 1 : 2);
        const int rows_wg = 16 * nr;
        const int tiles = cdiv(N, rows_wg);
        int chosen = -1;
        for (int s : kSplits) {
            if (!consider_split(s))
                continue;
            auto [per, eff] = split_chunks(KB, s, 16);
            if (split_req <= 0) {
                if (s > 1 && (eff < s || per < kMinSkinnyChunk))
                    break;  // chunks would collapse or be too short for their tail
                chosen = s;
                if ((int64_t)tiles * eff * 5 >= 4LL * num_cu)
                    break;
            } else {
                chosen = s;
            }
        }
        if (chosen < 0)
            chosen = 1;
        auto [per, eff] = split_chunks(KB, chosen, 16);
        best.family = 1;
        best.index = nri;
        best.bm = 16;
        best.bn = rows_wg;
        best.split = eff;
        best.kb_per_split = per;
        best.tiles_m = 1;
        best.tiles_n = tiles;
        best.grid = (int64_t)tiles * eff;
        best.name = skinny[best.index].name;
        const size_t part = (size_t)rows_wg * 16 * 4;
        best.counter_bytes = best.split > 1 ? (size_t)tiles * 4 : 0;
        best.ws_bytes = best.split > 1 ? (size_t)tiles * best.split * part : 0;
        return best;
    }

    int force_tile = -1;
    if (const char *e = std::getenv("MXGEMM_FORCE_TILE"))
        force_tile = std::atoi(e);
    for (int k = 0; k < n_tile; ++k) {
        if (force_tile >= 0 && force_tile < n_tile && k != force_tile)
            continue;
        const mx::TileKernel &tk = tile[k];
        const int tm = cdiv(M, tk.bm), tn = cdiv(N, tk.bn);
        const int64_t tiles = (int64_t)tm * tn;
        for (int s : kSplits) {
            if (!consider_split(s))
                continue;
            auto [per, eff] = split_chunks(KB, s, 8);
            if (split_req <= 0 && s > 1 && eff < s)
                continue;
            const int64_t wgs = tiles * eff;
            const int64_t slots = (int64_t)num_cu * tk.occupancy;
            const int64_t rounds = (wgs + slots - 1) / slots;
            // a single, partly filled round runs its stages faster
            const double fill = std::min(1.0, (double)wgs / (double)slots);
            const double ts = tile_stage_seconds(tk.bm, tk.bn) * (rounds == 1 ? 0.5 + 0.5 * fill : 1.0);
            double t = (double)rounds * (per / 8) * ts;
            if (eff > 1)
                t += kTileChunkCost * eff + (double)tiles * eff * tk.bm * tk.bn * 4 * 2 / kHbm +
                     (double)eff * tk.bm * tk.bn * 4 / kCuL2;
            // (on a tie the later candidate -- smaller tile, larger split --
            // wins: measured ties went to the one with more workgroups)
            if (t <= best_t * 1.005 || split_req > 0) {
                if (split_req > 0 && t >= best_t)
                    continue;
                best_t = t;
                best.family = 0;
                best.index = k;
                best.bm = tk.bm;
                best.bn = tk.bn;
                best.split = eff;
                best.kb_per_split = per;
                best.tiles_m = tm;
                best.tiles_n = tn;
                best.grid = wgs;
                best.name = tk.name;
            }
        }
    }
    const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
    best.counter_bytes = best.split > 1 ? (size_t)tiles * 4 : 0;
    best.ws_bytes = best.split > 1 ? (size_t)tiles * best.split * best.bm * best.bn * 4 : 0;
    return best;
}

// Tiled plan for 8-bit A (family 3): the cost model of the FP4 tiles with
// the matrix time doubled (the 8-bit scaled instruction runs at half the
// FP4 rate, "CDNA4 dense MFMA builtins", "Instruction throughput") and A's
// bytes doubled.  FP6 A (fp6 = true) keeps the FP4 matrix rate (the same
// table gives FP6 the FP4 cycles), in its padded 8-bit-sized layout or, on
// the dense FP6 tile, with 24 bytes per K-block (a row-major B is packed
// for it first, at the cost of a pass over B).
// MXGEMM_A8_TILE=<kernel name> restricts the choice to that tile where it
// applies (a test hook).
Plan plan_a8(int M, int N, int K, int split_req, int num_cu, bool fp6 = false, bool b_packed = false,
             bool dense_only = false)
{
    const int KB = K / 32;
    if (num_cu <= 0)
        num_cu = 256;
    int n = 0;
    const mx::TileKernelA8 *tile = mx::tile_kernels_a8(&n);
    const char *only = std::getenv("MXGEMM_A8_TILE");
    bool only_ok = false;
    for (int k = 0; only && k < n; ++k)
        only_ok |= std::strcmp(only, tile[k].name) == 0 && (!tile[k].fp6_dense || fp6);
    Plan best;
    double best_t = 1e300;
    for (int k = 0; k < n; ++k) {
        const mx::TileKernelA8 &tk = tile[k];
        if ((tk.fp6_dense && !fp6) || (dense_only && !tk.fp6_dense))
            continue;
        if (only_ok && std::strcmp(only, tk.name) != 0)
            continue;
        const double a_rows = tk.fp6_dense ? 1.5 : 2.0;  // A bytes per stage, in FP4 tile rows
        const int tm = cdiv(M, tk.bm), tn = cdiv(N, tk.bn);
        const int64_t tiles = (int64_t)tm * tn;
        for (int s : kSplits) {
            if (split_req > 0 && s != split_req)
                continue;
            auto [per, eff] = split_chunks(KB, s, 8);
            if (split_req <= 0 && s > 1 && eff < s)
                continue;
            const int64_t wgs = tiles * eff;
            const double rounds = (double)((wgs + (int64_t)num_cu * tk.occupancy - 1) / ((int64_t)num_cu * tk.occupancy));
            const double t_math = (fp6 ? 1.0 : 2.0) * 2.0 * tk.bm * tk.bn * 256.0 * tk.occupancy / (kCuFlops * kMatrixFraction);
            const double t_load = (a_rows * tk.bm + tk.bn) * 128.0 * tk.occupancy / kCuLoadRate;
            double t = rounds * (per / 8) * std::max(t_math, t_load);
            // the dense FP6 tile's stages run like the FP4 256 x 256 tile's:
            // 8192^3 in 314-316 us against 438-440 us on the 128 x 256
            // 8-bit tile, 4096^3 in 52.8 against 64.6-65.4 us (MI355X)
            if (tk.fp6_dense)
                t = t * 0.7 + (b_packed ? 0.0 : (double)N * K / kHbm);  // B's codes read and written once
            if (eff > 1)
                t += kSplitChunkCost * eff + (double)tiles * eff * tk.bm * tk.bn * 4 * 2 / kHbm +
                     (double)eff * tk.bm * tk.bn * 4 / kCuL2;
            if (t < best_t * 0.97 || (split_req > 0 && t < best_t)) {
                best_t = t;
                best.family = 3;
                best.index = k;
                best.bm = tk.bm;
                best.bn = tk.bn;
                best.split = eff;
                best.kb_per_split = per;
                best.tiles_m = tm;
                best.tiles_n = tn;
                best.grid = wgs;
                best.name = tk.name;
            }
        }
    }
    const int64_t tiles = (int64_t)best.tiles_m * best.tiles_n;
    best.counter_bytes = best.split > 1 ? (size_t)tiles * 4 : 0;
    best.ws_bytes = best.split > 1 ? (size_t)tiles * best.split * best.bm * best.bn * 4 : 0;
    return best;
}

// The plan mxgemm_run follows for these options: FP4 A by the cost model
// (the tiled kernel only in the bf16-atomic mode); a wider A with
// 16 < M <= 64 on the rows kernel (FP6: an even K-block count); otherwise
// with M > 16 on the 8-bit tiles, FP6 re-laid first; any other wider A at
// M == 1 on the single-row GEMV where it applies, else on the skinny kernel
// per 16 rows.
Plan plan_run(int M, int N, int K, const mxgemm_strides &s, int split_k, int num_cu, bool allow_gemv = true)
{
    // an MN-major B is read through the tiled kernel's transposed LDS loads
    if (s.a_format == MXGEMM_FMT_FP4)
        return plan_for(M, N, K, s.b_packed, split_k, num_cu,
                        s.split_mode == MXGEMM_SPLIT_BF16_ATOMIC || s.b_layout == MXGEMM_B_KN, 0,
                        MXGEMM_FMT_FP4, allow_gemv);
    const bool fp6 = s.a_format == MXGEMM_FMT_FP6_E2M3 || s.a_format == MXGEMM_FMT_FP6_E3M2;
    // an A already in the dense FP6 operand order (mxgemm_pack_a) is read
    // by the dense FP6 tile only
    if (fp6 && s.a_packed)
        return plan_a8(M, N, K, split_k, num_cu, true, s.b_packed != 0, true);
    if (M > 16 && M <= 64 && (!fp6 || (K / 32) % 2 == 0))
        return plan_for(M, N, K, s.b_packed, split_k, num_cu, false, 0, s.a_format);
    if ((s.a_format == MXGEMM_FMT_FP8_E4M3 || s.a_format == MXGEMM_FMT_FP8_E5M2) && M > 16)
        return plan_a8(M, N, K, split_k, num_cu);
    // FP6 with M > 16: A re-laid into 32-byte blocks (rows of K bytes rounded
    // up to 128), then the 8-bit tiles with the FP6 instruction, while a
    // 256-row tile of the re-laid A stays below 2^31 bytes
    if (fp6 && M > 16 && (int64_t)256 * mx::fp6_pad_pitch(K) < ((int64_t)1 << 31))
        return plan_a8(M, N, K, split_k, num_cu, true, s.b_packed != 0);
    return plan_for(std::min(M, 16), N, K, s.b_packed, split_k, num_cu, false, 1, s.a_format, allow_gemv);
}

size_t packed_b_bytes(int N, int K) { return (size_t)cdiv(N, 16) * 16 * (size_t)cdiv(K / 32, 4) * 64; }
size_t packed_sb_bytes(int N, int K) { return (size_t)cdiv(N, 32) * 32 * (size_t)cdiv(K / 32, 8) * 8; }

// The two-stage tiled kernel's 256 x 256 tile with packed A and B scales (B's
// codes packed or MN-major; or the dense FP6 tile) runs
// persistent (one workgroup per CU walking its tiles) when every tile is
// whole and unsplit, the epilogue is staged (d_stage), whole 8-block stages
// with 8-byte scale loads apply (svec), each tile has an even number of
// stages and there is more than one round of tiles.  Returns the persistent
// grid, or 0 for the plain grid.
int64_t persist_grid(const Plan &p, int M, int N, int K, int num_cu, bool d_stage, bool svec, bool sa_packed)
{
    const char *e = std::getenv("MXGEMM_TILE_PERSIST");  // "0": always the plain grid
    if (e && std::strcmp(e, "0") == 0)
        return 0;
    const char *pipe = std::getenv("MXGEMM_TILE_PIPELINE");
    if (pipe && std::strcmp(pipe, "deep") == 0)
        return 0;
    // (the dense FP6 tile, family 3's only 256 x 256 one, always reads
    // packed A scales)
    const bool tile_ok = p.bm == 256 && p.bn == 256 && ((p.family == 0 && sa_packed) || p.family == 3);
    if (!tile_ok || p.split != 1 || !d_stage || !svec)
        return 0;
    if (M % p.bm || N % p.bn || (K / 32) % 16 || num_cu % 8 || p.grid <= num_cu)
        return 0;
    return num_cu;
}

// ---- device facts, queried once per device

struct DeviceInfo {
    bool known = false;
    bool gfx950 = false;
    int num_cu = 0;
    double clock_hz = 0;
    char arch[32] = {0};
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_mutex;

mxgemm_status device_info(DeviceInfo **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return MXGEMM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo &d = g_dev[dev];
    if (!d.known) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess)
            return MXGEMM_ERR_HIP;
        std::snprintf(d.arch, sizeof d.arch, "%s", p.gcnArchName);
        d.gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
        d.num_cu = p.multiProcessorCount;
        d.clock_hz = (double)p.clockRate * 1e3;
        d.known = true;
    }
    *out = &d;
    return d.gfx950 ? MXGEMM_OK : MXGEMM_ERR_UNSUPPORTED_DEVICE;
}

// ---- library-owned split-K buffers, one set per (device, stream)
//
// Arrival counters live in a buffer of their own that only ever holds
// counters: it is zeroed when allocated and every kernel that increments a
// counter returns it to zero, so it is all zeros between calls whatever the
// previous plan was.  Partial sums live in a separate buffer (or in the
// caller's workspace), so stale partials can never be mistaken for counts.

struct DeviceBuffer {
    void *ptr = nullptr;
    size_t bytes = 0;
};
struct StreamBuffers {
    DeviceBuffer partials, counters;
    DeviceBuffer conv;  // FP6 A re-laid in 32-byte blocks (M x fp6_pad_pitch(K) bytes)
};
std::map<std::pair<int, hipStream_t>, StreamBuffers> g_ws;

mxgemm_status grow(DeviceBuffer &b, size_t need, hipStream_t stream, bool zero)
{
    if (b.bytes >= need)
        return MXGEMM_OK;
    if (b.ptr) {
        // earlier work on this stream may still use the old buffer
        if (hipStreamSynchronize(stream) != hipSuccess || hipFree(b.ptr) != hipSuccess)
            return MXGEMM_ERR_HIP;
        b.ptr = nullptr;
        b.bytes = 0;
    }
    const size_t sz = align_up(need, (size_t)1 << 16);
    void *p = nullptr;
    if (hipMalloc(&p, sz) != hipSuccess)
        return MXGEMM_ERR_HIP;
    if (zero) {
        // zeroed by a kernel on the caller's stream, so that the zeroing is
        // ordered before every later launch on that stream that uses the
        // buffer (a memset on the null stream is not ordered with
        // non-blocking streams)
        mx::launch_zero_words((uint32_t *)p, sz / 4, stream);
        if (hipGetLastError() != hipSuccess) {
            (void)hipFree(p);
            return MXGEMM_ERR_HIP;
        }
    }
    b.ptr = p;
    b.bytes = sz;
    return MXGEMM_OK;
}

// Counters (always library-owned) and, when part_need > 0, partials.
mxgemm_status get_split_buffers(hipStream_t stream, size_t counter_need, size_t part_need, void **counters,
                                void **partials)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MXGEMM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    StreamBuffers &w = g_ws[{dev, stream}];
    mxgemm_status st = grow(w.counters, counter_need, stream, true);
    if (st != MXGEMM_OK)
        return st;
    *counters = w.counters.ptr;
    if (part_need > 0) {
        st = grow(w.partials, part_need, stream, false);
        if (st != MXGEMM_OK)
            return st;
        *partials = w.partials.ptr;
    }
    return MXGEMM_OK;
}

// The per-stream buffer for FP6 A re-laid for the 8-bit tiles.
mxgemm_status get_conv_buffer(hipStream_t stream, size_t need, void **conv)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return MXGEMM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    StreamBuffers &w = g_ws[{dev, stream}];
    mxgemm_status st = grow(w.conv, need, stream, false);
    if (st != MXGEMM_OK)
        return st;
    *conv = w.conv.ptr;
    return MXGEMM_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

mxgemm_status check_shape(int M, int N, int K)
{
    if (M < 1 || N < 1 || K < 32 || K % 32 != 0 || K > kMaxK)
        return MXGEMM_ERR_SHAPE;
    return MXGEMM_OK;
}

bool valid_split(int s) { return s == 0 || s == -1 || s == 1 || s == 2 || s == 4 || s == 8 || s == 16; }

}  // namespace

extern "C" {

const char *mxgemm_status_string(mxgemm_status s)
{
    switch (s) {
    case MXGEMM_OK: return "ok";
    case MXGEMM_ERR_INVALID_ARG: return "invalid argument";
    case MXGEMM_ERR_SHAPE: return "unsupported shape";
    case MXGEMM_ERR_ALIGN: return "misaligned pointer or stride";
    case MXGEMM_ERR_UNSUPPORTED_DEVICE: return "device is not gfx950";
    case MXGEMM_ERR_HIP: return "HIP runtime error";
    case MXGEMM_ERR_WORKSPACE: return "workspace too small";
    case MXGEMM_ERR_SCRATCH: return "plan needs more than the fixed scratch of mxgemm_run_noalloc";
    default: return "unknown status";
    }
}

static void fill_info(const Plan &p, int M, int N, int K, int num_cu, const mxgemm_strides &s, mxgemm_info *out)
{
    std::memset(out, 0, sizeof *out);
    // what mxgemm_run launches for beta == 0 and 16-byte aligned pointers
    const int KB = K / 32;
    const bool dense6 = p.family == 3 && p.bm == 256;  // scales packed by the library
    const bool svec = KB % 8 == 0 && (dense6 || ((s.sa_packed || s.ldsa % 8 == 0) && (s.b_packed || s.ldsb % 8 == 0)));
    out->persist_grid = persist_grid(p, M, N, K, num_cu, s.ldd % 8 == 0, svec, s.sa_packed != 0);
    out->kernel = p.family;
    out->tile_m = p.bm;
    out->tile_n = p.bn;
    out->split_k = p.split;
    out->grid = p.grid;
    out->workspace_bytes = p.ws_bytes;
    out->packed_b_bytes = packed_b_bytes(N, K);
    out->packed_sb_bytes = packed_sb_bytes(N, K);
    out->packed_sa_bytes = packed_sb_bytes(M, K);
    out->num_cu = num_cu;
    std::snprintf(out->kernel_name, sizeof out->kernel_name, "%s", p.name);
}

mxgemm_status mxgemm_plan(int M, int N, int K, int b_packed, int split_k, int num_cu, mxgemm_info *out)
{
    if (!out || !valid_split(split_k) || (b_packed != 0 && b_packed != 1) || num_cu < 1)
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(M, N, K);
    if (st != MXGEMM_OK)
        return st;
    mxgemm_strides dense;
    std::memset(&dense, 0, sizeof dense);
    dense.ldd = N;
    dense.ldsa = dense.ldsb = K / 32;
    dense.b_packed = b_packed;
    fill_info(plan_for(M, N, K, b_packed, split_k, num_cu), M, N, K, num_cu, dense, out);
    return MXGEMM_OK;
}

static bool valid_options(const mxgemm_strides &s)
{
    return (s.b_packed == 0 || s.b_packed == 1) && (s.sa_packed == 0 || s.sa_packed == 1) &&
           (!s.sa_packed || s.b_packed) && (s.c_f32 == 0 || s.c_f32 == 1) &&
           (s.split_mode == MXGEMM_SPLIT_FP32 || s.split_mode == MXGEMM_SPLIT_BF16_ATOMIC) &&
           s.a_format >= MXGEMM_FMT_FP4 && s.a_format <= MXGEMM_FMT_FP6_E3M2 &&
           (s.b_layout == MXGEMM_B_NK || (s.b_layout == MXGEMM_B_KN && s.a_format == MXGEMM_FMT_FP4)) &&
           (s.a_format == MXGEMM_FMT_FP4 || (!s.sa_packed && s.split_mode == MXGEMM_SPLIT_FP32)) &&
           (s.a_packed == 0 ||
            (s.a_packed == 1 && (s.a_format == MXGEMM_FMT_FP6_E2M3 || s.a_format == MXGEMM_FMT_FP6_E3M2)));
}

mxgemm_status mxgemm_plan_ex(int M, int N, int K, const mxgemm_strides *strides, int split_k, int num_cu,
                             mxgemm_info *out)
{
    mxgemm_strides s;
    std::memset(&s, 0, sizeof s);
    if (strides)
        s = *strides;
    if (!out || !valid_split(split_k) || num_cu < 1 || !valid_options(s) || (s.a_packed && M <= 64))
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(M, N, K);
    if (st != MXGEMM_OK)
        return st;
    if (s.ldd == 0)
        s.ldd = N;
    if (s.ldsa == 0)
        s.ldsa = K / 32;
    if (s.ldsb == 0)
        s.ldsb = K / 32;
    fill_info(plan_run(M, N, K, s, split_k, num_cu), M, N, K, num_cu, s, out);
    return MXGEMM_OK;
}

mxgemm_status mxgemm_query_ex(int M, int N, int K, const mxgemm_strides *strides, int split_k, mxgemm_info *out)
{
    DeviceInfo *d = nullptr;
    if (!out)
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    st = mxgemm_plan_ex(M, N, K, strides, split_k, d->num_cu, out);
    if (st != MXGEMM_OK)
        return st;
    std::snprintf(out->arch, sizeof out->arch, "%s", d->arch);
    out->clock_hz = d->clock_hz;
    out->peak_flops = 65536.0 / 16.0 * 4.0 * d->num_cu * d->clock_hz;
    return MXGEMM_OK;
}

mxgemm_status mxgemm_query(int M, int N, int K, int b_packed, int split_k, mxgemm_info *out)
{
    if (!out || !valid_split(split_k) || (b_packed != 0 && b_packed != 1))
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(M, N, K);
    if (st != MXGEMM_OK)
        return st;
    DeviceInfo *d = nullptr;
    st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    st = mxgemm_plan(M, N, K, b_packed, split_k, d->num_cu, out);
    if (st != MXGEMM_OK)
        return st;
    std::snprintf(out->arch, sizeof out->arch, "%s", d->arch);
    out->clock_hz = d->clock_hz;
    // 16x16x128 FP4: 65536 flop per 16 cycles per matrix core ("CDNA4 dense
    // MFMA builtins", "Instruction throughput"), four matrix cores per CU.
    out->peak_flops = 65536.0 / 16.0 * 4.0 * d->num_cu * d->clock_hz;
    return MXGEMM_OK;
}

}  // extern "C"

namespace {

// mxgemm_run, and with X != NULL the fused single-row form of
// mxgemm_run_bf16a: A is the bf16 row X (ldx elements between rows),
// quantized to MXFP4 on load by the skinny kernel; A and scaleA are unused.
mxgemm_status run_impl(void *D, const void *C, const void *A, const void *B, const void *scaleA,
                       const void *scaleB, float alpha, float beta, int M, int N, int K,
                       const mxgemm_strides *strides, int split_k, hipStream_t stream, const void *X,
                       int64_t ldx, bool noalloc = false)
{
    // ---- host-only validation (no HIP call before it passes)
    if (!D || !B || !scaleB || !valid_split(split_k))
        return MXGEMM_ERR_INVALID_ARG;
    if (X ? M != 1 : (!A || !scaleA))
        return MXGEMM_ERR_INVALID_ARG;
    if (beta != 0.0f && !C)
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(M, N, K);
    if (st != MXGEMM_OK)
        return st;
    mxgemm_strides s;
    if (strides) {
        s = *strides;
        if ((s.b_packed != 0 && s.b_packed != 1) || (s.sa_packed != 0 && s.sa_packed != 1) ||
            (s.sa_packed && !s.b_packed) || (s.c_f32 != 0 && s.c_f32 != 1) ||
            (s.split_mode != MXGEMM_SPLIT_FP32 && s.split_mode != MXGEMM_SPLIT_BF16_ATOMIC) ||
            s.a_format < MXGEMM_FMT_FP4 || s.a_format > MXGEMM_FMT_FP6_E3M2 ||
            (s.b_layout != MXGEMM_B_NK && s.b_layout != MXGEMM_B_KN) ||
            (s.b_layout == MXGEMM_B_KN && s.a_format != MXGEMM_FMT_FP4))
            return MXGEMM_ERR_INVALID_ARG;
        if (s.a_format != MXGEMM_FMT_FP4 && (s.sa_packed || s.split_mode != MXGEMM_SPLIT_FP32))
            return MXGEMM_ERR_INVALID_ARG;
        // a pre-packed FP6 A feeds the dense FP6 tile, which runs for M > 64
        if ((s.a_packed != 0 && s.a_packed != 1) ||
            (s.a_packed && (X || M <= 64 || (s.a_format != MXGEMM_FMT_FP6_E2M3 && s.a_format != MXGEMM_FMT_FP6_E3M2))))
            return MXGEMM_ERR_INVALID_ARG;
        if (s.a_packed) {  // lda and ldsa are not used: the layout is fixed by M and K
            s.lda = K;
            s.ldsa = K / 32;
        }
    } else {
        std::memset(&s, 0, sizeof s);
        s.ldd = s.ldc = N;
        s.lda = s.ldb = K;
        s.ldsa = s.ldsb = K / 32;
    }
    const int KB = K / 32;
    if (X) {
        // the bf16 row replaces A and its scales
        if (s.a_format != MXGEMM_FMT_FP4 || s.sa_packed || s.split_mode != MXGEMM_SPLIT_FP32 ||
            s.b_layout != MXGEMM_B_NK)
            return MXGEMM_ERR_INVALID_ARG;
        if (ldx < K)
            return MXGEMM_ERR_SHAPE;
        if (!aligned(X, 16) || ldx % 8)
            return MXGEMM_ERR_ALIGN;
        A = X;
        s.lda = 4 * ldx;  // the row's byte pitch (2 * ldx) in fp4 elements
        s.ldsa = KB;
    }
    if (s.ldd < N || s.lda < K || (!s.sa_packed && s.ldsa < KB) || (beta != 0.0f && s.ldc < N))
        return MXGEMM_ERR_SHAPE;
    // B's codes as rows: [N][ldb/2] (K-major) or [K][ldb/2] (MN-major, whose
    // scales may still be packed)
    const bool b_kn = s.b_layout == MXGEMM_B_KN;
    const bool b_rows = !s.b_packed || b_kn;
    if ((b_kn ? s.ldb < N : (!s.b_packed && s.ldb < K)) || (!s.b_packed && s.ldsb < KB))
        return MXGEMM_ERR_SHAPE;
    // A's byte pitch: lda elements of its format (FP4: 4 bits, FP8: 8, FP6: 6)
    static const int kBits[5] = {4, 8, 8, 6, 6};
    const int a_bits = kBits[s.a_format];
    if ((s.lda * a_bits) % 8 || (b_rows && s.ldb % 2))
        return MXGEMM_ERR_ALIGN;
    const int64_t lda_bytes = s.lda * a_bits / 8;
    // (an FP6 row of K elements is 24 * K/32 bytes: its loads need 8-byte rows)
    if (!aligned(A, 16) || !aligned(B, 16) || lda_bytes % (a_bits == 6 ? 8 : 16) ||
        (b_rows && (s.ldb / 2) % 16))
        return MXGEMM_ERR_ALIGN;
    if ((s.b_packed && !aligned(scaleB, 4)) || (!X && (s.sa_packed || s.a_packed) && !aligned(scaleA, 4)))
        return MXGEMM_ERR_ALIGN;
    if (!aligned(D, 2) || (C && beta != 0.0f && !aligned(C, s.c_f32 ? 4 : 2)))
        return MXGEMM_ERR_ALIGN;
    const bool atomic = s.split_mode == MXGEMM_SPLIT_BF16_ATOMIC;
    if (atomic && (!aligned(D, 4) || s.ldd % 2 || N % 2))
        return MXGEMM_ERR_ALIGN;
    // byte offsets and buffer ranges inside a 256-row tile must stay below
    // 2^31: A and B rows, scale rows, and a 256-row slice of packed B
    const int64_t k31 = (int64_t)1 << 31;
    if ((int64_t)256 * lda_bytes >= k31 || (b_rows && (int64_t)256 * (s.ldb / 2) >= k31) ||
        (!X && !s.sa_packed && (int64_t)256 * s.ldsa >= k31) || (!s.b_packed && (int64_t)256 * s.ldsb >= k31) ||
        (s.b_packed && !b_kn && (int64_t)16 * cdiv(KB, 4) * 1024 >= k31))
        return MXGEMM_ERR_SHAPE;

    // ---- device and plan
    DeviceInfo *d = nullptr;
    st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    // the GEMV reads the scale rows as aligned dwords (16-byte aligned rows,
    // as the skinny kernel's vector scale path).  A bf16 A row stays on the
    // skinny kernel's quantize-on-load: the GEMV's 4-row workgroups would
    // each load and encode the whole row (2048 times at N = 8192, 32 MiB of
    // bf16 from L2), which measured 10.2-10.4 us against 8.8 us
    const bool gemv_ok = !X && aligned(scaleA, 16) && s.ldsa % 16 == 0 && aligned(scaleB, 16) && s.ldsb % 16 == 0;
    Plan p = plan_run(M, N, K, s, split_k, d->num_cu, gemv_ok);
    // a wider A on the skinny kernel (one 16-row group, nr 1): one launch
    // per 16 rows of A
    const bool wide = s.a_format != MXGEMM_FMT_FP4 && p.family == 1;

    GemmArgs g;
    std::memset(&g, 0, sizeof g);
    g.D = (uint16_t *)D;
    g.C = C;
    g.A = (const uint8_t *)A;
    g.B = (const uint8_t *)B;
    g.SA = X ? nullptr : (const uint8_t *)scaleA;
    g.SB = (const uint8_t *)scaleB;
    g.alpha = alpha;
    g.beta = beta;
    g.M = M;
    g.N = N;
    g.K = K;
    g.KB = KB;
    g.lda_b = lda_bytes;
    g.ldb_b = s.ldb / 2;
    g.ldsa = s.ldsa;
    g.ldsb = s.ldsb;
    g.ldc = s.ldc;
    g.ldd = s.ldd;
    g.split = p.split;
    g.kb_per_split = p.kb_per_split;
    g.tiles_m = p.tiles_m;
    g.tiles_n = p.tiles_n;
    g.ks_total = cdiv(KB, 4);
    g.sn8 = cdiv(KB, 8);
    g.sa_fast = !X && aligned(scaleA, 8) && s.ldsa % 8 == 0 && KB % 8 == 0;
    g.sb_fast = !s.b_packed && aligned(scaleB, 8) && s.ldsb % 8 == 0 && KB % 8 == 0;
    g.scale16 = (X || (aligned(scaleA, 16) && s.ldsa % 16 == 0)) && KB % 16 == 0 &&
                (s.b_packed || (aligned(scaleB, 16) && s.ldsb % 16 == 0));
    g.d_vec = aligned(D, 8) && s.ldd % 4 == 0;
    g.c_vec = C && aligned(C, s.c_f32 ? 16 : 8) && s.ldc % 4 == 0;
    g.c_f32 = s.c_f32;
    g.d_stage = beta == 0.0f && aligned(D, 16) && s.ldd % 8 == 0;
    g.sa_packed = s.sa_packed;
    g.sa16 = !X && !s.sa_packed && aligned(scaleA, 16) && s.ldsa % 16 == 0 && KB % 16 == 0;
    g.sb16 = !s.b_packed && aligned(scaleB, 16) && s.ldsb % 16 == 0 && KB % 16 == 0;
    g.group_m = 4;

    // FP6 A on the 8-bit tiles is first re-laid into 32-byte blocks; on the
    // dense FP6 tile into its operand order, with the A scales shuffled
    // behind it
    const bool fp6_conv = p.family == 3 && (s.a_format == MXGEMM_FMT_FP6_E2M3 || s.a_format == MXGEMM_FMT_FP6_E3M2);
    int n_a8 = 0;
    const bool fp6_dense = fp6_conv && mx::tile_kernels_a8(&n_a8)[p.index].fp6_dense;
    // (a pre-packed A is read where it is: no copy of A or its scales)
    const bool a_here = fp6_dense && !s.a_packed;
    const size_t a6_bytes = a_here ? align_up((size_t)cdiv(M, 16) * (size_t)mx::fp6_pack_group_bytes(K), 256) : 0;
    // [A dense | A scales packed | B packed | B scales packed]: a row-major
    // B is packed too, the tile reads only the packed layout
    const bool pack_b_here = fp6_dense && !s.b_packed;
    const size_t sap_bytes = a_here ? align_up(packed_sb_bytes(M, K), 256) : 0;
    const size_t bp_bytes = pack_b_here ? align_up(packed_b_bytes(N, K), 256) : 0;
    const size_t conv_bytes = !fp6_conv ? 0
                              : fp6_dense ? a6_bytes + sap_bytes + bp_bytes + (pack_b_here ? packed_sb_bytes(N, K) : 0)
                                          : (size_t)M * (size_t)mx::fp6_pad_pitch(K);
    // the allocation-free form: counters, partials and the FP6 copy come
    // from the device's fixed scratch (counters first, then partials, then
    // the copy); a plan that needs more is refused before any launch
    uint8_t *scr = nullptr;
    size_t scr_part = 0;
    if (noalloc) {
        const bool fp32_split = p.split > 1 && !atomic;
        const size_t part = fp32_split && !s.workspace ? align_up(p.ws_bytes, 256) : 0;
        if ((fp32_split && p.counter_bytes > mx::kScratchCounterBytes) ||
            part + conv_bytes > mx::kScratchBytes - mx::kScratchCounterBytes)
            return MXGEMM_ERR_SCRATCH;
        void *base = nullptr;
        if (mx::scratch_address(&base) != hipSuccess)
            return MXGEMM_ERR_HIP;
        scr = (uint8_t *)base;
        scr_part = part;
    }

    if (p.split > 1 && atomic) {
        // chunks add into D, set first to bf16(beta * C); no workspace
        if ((int64_t)M * (N / 2) / 256 >= 0x7FFFFFFF)
            return MXGEMM_ERR_SHAPE;
        g.split_atomic = 1;
    } else if (p.split > 1) {
        void *counters = nullptr, *partials = nullptr;
        if (s.workspace && s.workspace_bytes < p.ws_bytes)
            return MXGEMM_ERR_WORKSPACE;
        if (noalloc) {
            // the scratch keeps the last call's contents: this call's
            // counters are cleared (by a kernel, ordered on `stream`)
            counters = scr;
            partials = scr + mx::kScratchCounterBytes;
            mx::launch_zero_words((uint32_t *)counters, (p.counter_bytes + 3) / 4, stream);
        } else {
            st = get_split_buffers(stream, p.counter_bytes, s.workspace ? 0 : p.ws_bytes, &counters, &partials);
            if (st != MXGEMM_OK)
                return st;
        }
        g.counters = (int *)counters;
        g.ws = (float *)(s.workspace ? s.workspace : partials);
    }

    if (p.grid > 0x7FFFFFFF)
        return MXGEMM_ERR_SHAPE;
    if (g.split_atomic)
        mx::launch_d_init(g, stream);
    if (X) {
        if (p.family != 1)  // M == 1 with the fp32 split reduction plans the skinny kernel
            return MXGEMM_ERR_INVALID_ARG;
        mx::launch_skinny_bf16a(p.bn / 16, s.b_packed != 0, g, (int)p.grid, stream);
    } else if (wide) {
        // stream-ordered launches over 16-row blocks of A, C and D; the split
        // counters return to zero at the end of each
        for (int m0 = 0; m0 < M; m0 += 16) {
            GemmArgs gb = g;
            gb.M = std::min(16, M - m0);
            gb.A = g.A + (int64_t)m0 * g.lda_b;
            gb.SA = g.SA + (int64_t)m0 * g.ldsa;
            gb.D = g.D + (int64_t)m0 * g.ldd;
            if (g.C)
                gb.C = (const uint8_t *)g.C + (int64_t)m0 * g.ldc * (g.c_f32 ? 4 : 2);
            mx::launch_skinny_wide(s.a_format, s.b_packed != 0, gb, (int)p.grid, stream);
        }
    } else if (p.family == 3) {
        int n = 0;
        const mx::TileKernelA8 &k = mx::tile_kernels_a8(&n)[p.index];
        if (fp6_conv) {
            // FP6 A re-laid into the 8-bit operand shape, codes and scales unchanged
            void *conv = nullptr;
            if (noalloc) {
                conv = scr + mx::kScratchCounterBytes + scr_part;
            } else if (conv_bytes > 0) {
                st = get_conv_buffer(stream, conv_bytes, &conv);
                if (st != MXGEMM_OK)
                    return st;
            }
            if (fp6_dense) {
                uint8_t *sap = (uint8_t *)conv + a6_bytes;
                if (a_here) {
                    mx::launch_fp6_pack((const uint8_t *)A, lda_bytes, (const uint8_t *)scaleA, s.ldsa,
                                        (uint8_t *)conv, (uint32_t *)sap, M, K, stream);
                    g.A = (const uint8_t *)conv;
                    g.SA = sap;
                } else {  // mxgemm_pack_a's output, read in place
                    g.A = (const uint8_t *)A;
                    g.SA = (const uint8_t *)scaleA;
                }
                g.lda_b = mx::fp6_pack_group_bytes(K);
                g.sa_packed = 1;
                g.persist_grid = (int)persist_grid(p, M, N, K, d->num_cu, g.d_stage != 0, KB % 8 == 0, true);
                if (pack_b_here) {
                    uint8_t *bp = sap + sap_bytes, *sbp = bp + bp_bytes;
                    mx::launch_pack_b(bp, (const uint8_t *)B, N, KB, s.ldb / 2, stream);
                    mx::launch_pack_sb((uint32_t *)sbp, (const uint8_t *)scaleB, N, KB, s.ldsb, stream);
                    g.B = bp;
                    g.SB = sbp;
                }
            } else {
                mx::launch_fp6_pad((const uint8_t *)A, lda_bytes, (uint8_t *)conv, M, K, stream);
                g.A = (const uint8_t *)conv;
                g.lda_b = mx::fp6_pad_pitch(K);
            }
        }
        (s.b_packed || fp6_dense ? k.packed : k.plain)[s.a_format - 1](g, (int)p.grid, stream);
    } else if (p.family == 0) {
        int n = 0;
        const mx::TileKernel &k = mx::tile_kernels(&n)[p.index];
        // the four-slot ring kernel moves scales as 4-byte words and whole
        // 128-K steps; otherwise the two-stage kernel handles any layout
        const bool deep_ok = KB % 4 == 0 && (s.sa_packed || (aligned(scaleA, 4) && s.ldsa % 4 == 0)) &&
                             (s.b_packed || (aligned(scaleB, 4) && s.ldsb % 4 == 0));
        bool deep = deep_ok && k.prefer_deep && !g.split_atomic && !b_kn;  // the two-stage kernel implements
                                                                           // the atomic mode and MN-major B
        if (const char *e = std::getenv("MXGEMM_TILE_PIPELINE")) {  // "deep" or "two-stage"
            if (std::strcmp(e, "two-stage") == 0)
                deep = false;
            else if (std::strcmp(e, "deep") == 0)
                deep = deep_ok && !g.split_atomic && !b_kn;
        }
        if (!deep) {
            const bool svec = (s.sa_packed ? KB % 8 == 0 : g.sa_fast != 0) &&
                              (s.b_packed ? KB % 8 == 0 : g.sb_fast != 0);
            g.persist_grid = (int)persist_grid(p, M, N, K, d->num_cu, g.d_stage != 0, svec, s.sa_packed != 0);
        }
        if (b_kn)
            (s.sa_packed ? k.kn_packed_sa : s.b_packed ? k.kn_packed_sb : k.kn)(g, (int)p.grid, stream);
        else if (deep)
            (s.sa_packed ? k.deep_packed_sa : s.b_packed ? k.deep_packed : k.deep_plain)(g, (int)p.grid, stream);
        else
            (s.sa_packed ? k.packed_sa : s.b_packed ? k.packed : k.plain)(g, (int)p.grid, stream);
    } else if (p.family == 4) {
        mx::launch_gemv(s.a_format, g, (int)p.grid, stream);
    } else if (p.family == 1) {
        int n = 0;
        const mx::SkinnyKernel &k = mx::skinny_kernels(&n)[p.index];
        (s.sa_packed ? k.packed_sa : s.b_packed ? k.packed : k.plain)(g, (int)p.grid, stream);
    } else {
        int n = 0;
        const mx::RowsKernel &k = mx::rows_kernels(&n)[p.index];
        (s.b_packed ? k.packed[s.a_format] : p.lean ? k.lean : k.plain[s.a_format])(g, (int)p.grid, stream);
    }
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

}  // namespace

extern "C" {

mxgemm_status mxgemm_run(void *D, const void *C, const void *A, const void *B, const void *scaleA,
                         const void *scaleB, float alpha, float beta, int M, int N, int K,
                         const mxgemm_strides *strides, int split_k, hipStream_t stream)
{
    return run_impl(D, C, A, B, scaleA, scaleB, alpha, beta, M, N, K, strides, split_k, stream, nullptr, 0);
}

mxgemm_status mxgemm_run_noalloc(void *D, const void *C, const void *A, const void *B, const void *scaleA,
                                 const void *scaleB, float alpha, float beta, int M, int N, int K,
                                 const mxgemm_strides *strides, int split_k, hipStream_t stream)
{
    return run_impl(D, C, A, B, scaleA, scaleB, alpha, beta, M, N, K, strides, split_k, stream, nullptr, 0, true);
}

mxgemm_status mxgemm_run_bf16a(void *D, const void *C, const void *X, const void *B, const void *scaleB,
                               float alpha, float beta, int M, int N, int K, int64_t ldx,
                               const mxgemm_strides *strides, int split_k, hipStream_t stream)
{
    if (!X)
        return MXGEMM_ERR_INVALID_ARG;
    // the fused decode kernel streams a K-major B; an MN-major B goes through
    // the tiled kernel like M > 1
    if (M == 1 && !(strides && strides->b_layout == MXGEMM_B_KN))
        return run_impl(D, C, nullptr, B, nullptr, scaleB, alpha, beta, M, N, K, strides, split_k, stream, X, ldx);
    // M > 1: quantize into a per-stream buffer, then the ordinary call
    mxgemm_status st = check_shape(M, N, K);
    if (st != MXGEMM_OK)
        return st;
    if (strides && (strides->a_format != MXGEMM_FMT_FP4 || strides->sa_packed))
        return MXGEMM_ERR_INVALID_ARG;
    const size_t a_bytes = align_up((size_t)M * (size_t)(K / 2), 256);
    void *buf = nullptr;
    st = get_conv_buffer(stream, a_bytes + (size_t)M * (size_t)(K / 32), &buf);
    if (st != MXGEMM_OK)
        return st;
    uint8_t *Aq = (uint8_t *)buf, *SAq = Aq + a_bytes;
    st = mxgemm_quantize(Aq, SAq, X, M, K, ldx, K, K / 32, stream);
    if (st != MXGEMM_OK)
        return st;
    mxgemm_strides s2;
    if (strides) {
        s2 = *strides;
    } else {
        std::memset(&s2, 0, sizeof s2);
        s2.ldd = s2.ldc = N;
        s2.ldb = K;
        s2.ldsb = K / 32;
    }
    s2.lda = K;
    s2.ldsa = K / 32;
    return mxgemm_run(D, C, Aq, B, SAq, scaleB, alpha, beta, M, N, K, &s2, split_k, stream);
}

mxgemm_status mxgemm_pack_b(void *Bp, void *SBp, const void *B, const void *scaleB, int N, int K, int64_t ldb,
                            int64_t ldsb, hipStream_t stream)
{
    if (!Bp || !SBp || !B || !scaleB)
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(1, N, K);
    if (st != MXGEMM_OK)
        return st;
    if (ldb < K || ldsb < K / 32)
        return MXGEMM_ERR_SHAPE;
    if (ldb % 2 || (ldb / 2) % 16 || !aligned(B, 16) || !aligned(Bp, 16) || !aligned(SBp, 4))
        return MXGEMM_ERR_ALIGN;
    DeviceInfo *d = nullptr;
    st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    mx::launch_pack_b((uint8_t *)Bp, (const uint8_t *)B, N, K / 32, ldb / 2, stream);
    mx::launch_pack_sb((uint32_t *)SBp, (const uint8_t *)scaleB, N, K / 32, ldsb, stream);
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

mxgemm_status mxgemm_pack_scales(void *Sp, const void *S, int rows, int K, int64_t lds, hipStream_t stream)
{
    if (!Sp || !S)
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(rows, 1, K);
    if (st != MXGEMM_OK)
        return st;
    if (lds < K / 32)
        return MXGEMM_ERR_SHAPE;
    if (!aligned(Sp, 4))
        return MXGEMM_ERR_ALIGN;
    DeviceInfo *d = nullptr;
    st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    mx::launch_pack_sb((uint32_t *)Sp, (const uint8_t *)S, rows, K / 32, lds, stream);
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

size_t mxgemm_pack_a_bytes(int M, int K)
{
    if (check_shape(M, 1, K) != MXGEMM_OK)
        return 0;
    return (size_t)cdiv(M, 16) * (size_t)mx::fp6_pack_group_bytes(K);
}

mxgemm_status mxgemm_pack_a(void *Ap, void *SAp, const void *A, const void *scaleA, int M, int K, int64_t lda,
                            int64_t ldsa, int a_format, hipStream_t stream)
{
    if (!Ap || !SAp || !A || !scaleA ||
        (a_format != MXGEMM_FMT_FP6_E2M3 && a_format != MXGEMM_FMT_FP6_E3M2))
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(M, 1, K);
    if (st != MXGEMM_OK)
        return st;
    if (lda < K || ldsa < K / 32)
        return MXGEMM_ERR_SHAPE;
    // FP6 rows: lda * 6 / 8 bytes, in whole 8-byte units, as mxgemm_run reads them
    if ((lda * 6) % 8 || (lda * 6 / 8) % 8 || !aligned(A, 16) || !aligned(Ap, 16) || !aligned(SAp, 4))
        return MXGEMM_ERR_ALIGN;
    DeviceInfo *d = nullptr;
    st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    mx::launch_fp6_pack((const uint8_t *)A, lda * 6 / 8, (const uint8_t *)scaleA, ldsa, (uint8_t *)Ap,
                        (uint32_t *)SAp, M, K, stream);
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

mxgemm_status mxgemm_f16_run(void *C, const void *A, const void *B, int M, int N, int K, int64_t lda,
                             int64_t ldb, int64_t ldc, hipStream_t stream)
{
    if (!C || !A || !B)
        return MXGEMM_ERR_INVALID_ARG;
    if (M < 1 || N < 1 || K < 1 || K % 8 || N % 8 || lda < K || ldb < N || ldc < N)
        return MXGEMM_ERR_SHAPE;
    if ((int64_t)256 * lda * 2 >= ((int64_t)1 << 31) || (int64_t)K * ldb * 2 >= ((int64_t)1 << 31))
        return MXGEMM_ERR_SHAPE;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 4) || lda % 8 || ldb % 8)
        return MXGEMM_ERR_ALIGN;
    DeviceInfo *d = nullptr;
    mxgemm_status st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    mx::F16Args a;
    std::memset(&a, 0, sizeof a);
    a.A = (const uint8_t *)A;
    a.B = (const uint8_t *)B;
    a.C = (float *)C;
    a.M = M;
    a.N = N;
    a.K = K;
    a.lda_b = lda * 2;
    a.ldb_b = ldb * 2;
    a.ldc = ldc;
    a.tiles_m = cdiv(M, 256);
    a.tiles_n = cdiv(N, 256);
    const int64_t grid = mx::f16_grid(M, N);
    if (grid > 0x7FFFFFFF)
        return MXGEMM_ERR_SHAPE;
    mx::launch_f16(a, grid, stream);
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

mxgemm_status mxgemm_quantize(void *A, void *scaleA, const void *X, int M, int K, int64_t ldx,
                              int64_t lda, int64_t ldsa, hipStream_t stream)
{
    if (!A || !scaleA || !X)
        return MXGEMM_ERR_INVALID_ARG;
    mxgemm_status st = check_shape(M, 1, K);
    if (st != MXGEMM_OK)
        return st;
    if (ldx < K || lda < K || ldsa < K / 32)
        return MXGEMM_ERR_SHAPE;
    // 16-byte loads of 8 bf16 per lane; A as mxgemm_run requires it
    if (lda % 2 || !aligned(X, 16) || ldx % 8 || !aligned(A, 16) || (lda / 2) % 16)
        return MXGEMM_ERR_ALIGN;
    const int64_t blocks = (int64_t)M * (K / 32);
    const int64_t grid = mx::quant_grid(blocks);
    if (grid > 0x7FFFFFFF)
        return MXGEMM_ERR_SHAPE;
    DeviceInfo *d = nullptr;
    st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    mx::QuantArgs q;
    q.X = (const uint16_t *)X;
    q.A = (uint8_t *)A;
    q.S = (uint8_t *)scaleA;
    q.M = M;
    q.K = K;
    q.ldx = ldx;
    q.lda_b = lda / 2;
    q.lds = ldsa;
    q.blocks = blocks;
    mx::launch_quant(q, grid, stream);
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

mxgemm_status mxgemm_stream_read(const void *src, size_t bytes, void *sink, hipStream_t stream)
{
    if (!src || !sink)
        return MXGEMM_ERR_INVALID_ARG;
    if (bytes == 0 || bytes % 16 || bytes >= ((size_t)1 << 31))
        return MXGEMM_ERR_SHAPE;
    if (!aligned(src, 16) || !aligned(sink, 4))
        return MXGEMM_ERR_ALIGN;
    DeviceInfo *d = nullptr;
    mxgemm_status st = device_info(&d);
    if (st != MXGEMM_OK)
        return st;
    mx::launch_stream_read((const uint8_t *)src, bytes, (uint32_t *)sink, stream);
    if (hipGetLastError() != hipSuccess)
        return MXGEMM_ERR_HIP;
    return MXGEMM_OK;
}

mxgemm_status mxgemm_release_workspaces(void)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    mxgemm_status st = MXGEMM_OK;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto &kv : g_ws) {
        if (hipSetDevice(kv.first.first) != hipSuccess || hipStreamSynchronize(kv.first.second) != hipSuccess)
            st = MXGEMM_ERR_HIP;
        for (DeviceBuffer *b : {&kv.second.partials, &kv.second.counters, &kv.second.conv})
            if (b->ptr && hipFree(b->ptr) != hipSuccess)
                st = MXGEMM_ERR_HIP;
    }
    (void)hipSetDevice(cur);
    g_ws.clear();
    return st;
}

}  // extern "C"
