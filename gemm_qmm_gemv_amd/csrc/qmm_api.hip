// qmm_api.hip -- the C ABI of libqmm: argument checks, launch planning and
// kernel launches.  Declarations and the contract are in include/qmm.h.
//
// Launch planning follows the pages' note that kernel choice and work-group
// sizes are tuned per chip and per GPU-core count ("BaseRT: Best-in-Class
// LLM Inference on Apple Silicon via Native Metal", section "Metodologia"):
// here the inputs are the shape, the bit width and the device's compute-unit
// count.  Everything is decided on the host from integers; no allocation,
// no synchronization, no per-call state.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <climits>
#include <cstring>
#include <mutex>

#include "../../include/qmm.h"
#include "qmm_kernels.h"

using namespace qmm;

namespace {

#define QMM_BITS_SWITCH(bits, FN, ...)                    \
    switch (bits) {                                       \
        case 2: return FN<2>(__VA_ARGS__);                \
        case 3: return FN<3>(__VA_ARGS__);                \
        case 4: return FN<4>(__VA_ARGS__);                \
        case 5: return FN<5>(__VA_ARGS__);                \
        case 6: return FN<6>(__VA_ARGS__);                \
        case 8: return FN<8>(__VA_ARGS__);                \
        case 16: return FN<16>(__VA_ARGS__);              \
        default: return hipErrorInvalidValue;             \
    }

hipError_t launch_gemv(const GemvArgs& a, const GemvShape& sh, hipStream_t st) {
    QMM_BITS_SWITCH(a.bits, launch_gemv_bits, a, sh, st)
}
hipError_t launch_batched(const BatchArgs& a, const GemvShape& sh, hipStream_t st) {
    QMM_BITS_SWITCH(a.bits, launch_batched_bits, a, sh, st)
}
hipError_t launch_rows(const RowsArgs& a, const RowsShape& sh, hipStream_t st) {
    QMM_BITS_SWITCH(a.bits, launch_rows_bits, a, sh, st)
}
hipError_t launch_glu(const GluArgs& a, const GemvShape& sh, hipStream_t st) {
    QMM_BITS_SWITCH(a.bits, launch_glu_bits, a, sh, st)
}

thread_local char g_err[512] = "";

qmm_status fail(qmm_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

qmm_status ok() {
    g_err[0] = '\0';
    return QMM_OK;
}

bool bits_supported(int bits) {
    return bits == 2 || bits == 3 || bits == 4 || bits == 5 || bits == 6 || bits == 8 || bits == 16;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t INT_LIMIT = 0x7fffffff;
constexpr int64_t OFFSET_LIMIT = 0xffffffffLL;  // largest byte size a 32-bit offset covers

qmm_status check_format(int64_t n, int64_t k, int bits, int group) {
    if (bits != 16 && (bits < 2 || bits > 8))
        return fail(QMM_ERR_INVALID_ARGUMENT, "bits=%d is neither 2..8 nor 16 (fp16)", bits);
    if (!bits_supported(bits))
        return fail(QMM_ERR_UNSUPPORTED, "bits=%d not built (supported: 2, 3, 4, 5, 6, 8, 16)", bits);
    if (group <= 0 || group % 32)
        return fail(QMM_ERR_INVALID_ARGUMENT, "group_size=%d must be a positive multiple of 32", group);
    if (k < 32 || k % group)
        return fail(QMM_ERR_INVALID_ARGUMENT, "k=%lld must be >= 32 and a multiple of group_size=%d",
                    (long long)k, group);
    if (n < 0) return fail(QMM_ERR_INVALID_ARGUMENT, "n=%lld is negative", (long long)n);
    if (n > INT_LIMIT || k > INT_LIMIT)
        return fail(QMM_ERR_INVALID_ARGUMENT, "n or k above 2^31-1");
    // The kernels address one matrix (and one activation block) with 32-bit
    // buffer offsets.
    if (n * (k / 32) * bits * 4 > OFFSET_LIMIT)
        return fail(QMM_ERR_UNSUPPORTED, "packed matrix of %lld x %lld at %d bits is 4 GiB or more",
                    (long long)n, (long long)k, bits);
    return QMM_OK;
}

qmm_status check_output_bytes(int64_t rows, int64_t n) {
    if (rows * n * 4 > OFFSET_LIMIT)
        return fail(QMM_ERR_UNSUPPORTED, "output of %lld x %lld fp32 is 4 GiB or more",
                    (long long)rows, (long long)n);
    return QMM_OK;
}

qmm_status check_activation_bytes(int64_t rows, int64_t k) {
    if (rows * k * 2 > OFFSET_LIMIT)
        return fail(QMM_ERR_UNSUPPORTED, "activation block of %lld x %lld fp16 is 4 GiB or more",
                    (long long)rows, (long long)k);
    return QMM_OK;
}

// fp16 weights (bits 16) have no scales or mins: those pointers are not read
// and may be NULL.
qmm_status check_weight_ptrs(const void* w, const void* s, const void* m, int bits) {
    if (!w) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL weight pointer");
    if (!aligned(w, 16)) return fail(QMM_ERR_MISALIGNED, "w_packed not 16-byte aligned");
    if (bits == 16) return QMM_OK;
    if (!s || !m) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL scale or min pointer");
    if (!aligned(s, 2) || !aligned(m, 2)) return fail(QMM_ERR_MISALIGNED, "scales/mins not 2-byte aligned");
    return QMM_OK;
}


// Compute units of the current device, cached per device id.
std::atomic<int> g_cu_cache[64];

qmm_status device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(QMM_ERR_DEVICE, "no HIP device available");
    }
    if (dev >= 0 && dev < 64) {
        const int c = g_cu_cache[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return QMM_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) {
        (void)hipGetLastError();
        return fail(QMM_ERR_DEVICE, "cannot query compute units of device %d", dev);
    }
    if (dev >= 0 && dev < 64) g_cu_cache[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return QMM_OK;
}

// Launch-plan overrides (measurement sweeps, tests that force a variant).
// They are read from the environment once, when the library is loaded, and
// changed in-process only through qmm_set_override: a call never reads the
// environment.  A negative value means "no override".
enum OverrideId {
    OV_UNIT, OV_GEMV_LPR, OV_GEMV_XC, OV_GEMV_U, OV_GEMV_WAVES_PER_CU, OV_BATCH_U, OV_ROWS_MR,
    OV_ROWS_WAVES_PER_CU, OV_GEMM_TILE_M, OV_GEMM_TILE_N, OV_GEMM_SPLIT, OV_GEMM_WIDE_SCALES,
    OV_GEMM_ORDER, OV_GEMM_GROUPED, OV_GEMM_KERNEL, OV_GEMV_STAGED, OV_GEMV_LATE, OV_COUNT
};
const char* const OVERRIDE_NAMES[OV_COUNT] = {
    "QMM_UNIT", "QMM_GEMV_LPR", "QMM_GEMV_XC", "QMM_GEMV_U", "QMM_GEMV_WAVES_PER_CU", "QMM_BATCH_U",
    "QMM_ROWS_MR", "QMM_ROWS_WAVES_PER_CU", "QMM_GEMM_TILE_M", "QMM_GEMM_TILE_N", "QMM_GEMM_SPLIT",
    "QMM_GEMM_WIDE_SCALES", "QMM_GEMM_ORDER", "QMM_GEMM_GROUPED", "QMM_GEMM_KERNEL", "QMM_GEMV_STAGED",
    "QMM_GEMV_LATE"};
std::atomic<int> g_override[OV_COUNT];

struct OverridesFromEnvironment {
    OverridesFromEnvironment() {
        for (int i = 0; i < OV_COUNT; ++i) {
            const char* v = getenv(OVERRIDE_NAMES[i]);
            g_override[i].store(v && *v ? atoi(v) : -1, std::memory_order_relaxed);
        }
    }
} g_overrides_at_load;

int override_or(OverrideId id, int dflt) {
    const int v = g_override[id].load(std::memory_order_relaxed);
    return v >= 0 ? v : dflt;
}

// Codes per activation unit: 64 when the group allows; fp16 weights use 32
// (a 64-code unit would be 32 weight words per lane and row).
int unit_codes(int bits, int group) {
    return (bits != 16 && group % 64 == 0 && override_or(OV_UNIT, 64) != 32) ? 64 : 32;
}

// ---- planning ------------------------------------------------------------------

struct LaneSplit {
    int lpr, xc;
    bool multipass;
};

// Lanes per row and units per lane.  One unit per lane while a row has at
// most 64 units (lanes = the next power of two: idle lanes cost less than a
// second serial unit, which doubles the activation registers and the work
// between a lane's loads); above that, 64 lanes with ceil(units/64) units each
// up to max_xc, and multi-pass beyond.
LaneSplit choose_split(int nu, int max_xc, bool (*supported)(int, int)) {
    int lpr = 16;
    while (lpr < 64 && lpr < nu) lpr *= 2;
    const int xc = (nu + lpr - 1) / lpr;
    if (xc <= max_xc && supported(lpr, xc)) return {lpr, xc, false};
    const int mxc = max_xc >= 2 ? 2 : 1;
    return {64, mxc, true};
}

bool gemv_split_ok(int lpr, int xc) { return gemv_shape_supported(lpr, xc, 1); }
bool rows_split_ok(int lpr, int xc) { return rows_shape_supported(lpr, xc, 1); }

GemvShape plan_gemv(int64_t n, int64_t k, int bits, int group, int cus) {
    GemvShape sh{};
    sh.unit = unit_codes(bits, group);
    const int nu = (int)(k / sh.unit);
    LaneSplit ls = choose_split(nu, 3, gemv_split_ok);
    // Rows of 33 to 48 units (K = 3072 at 64-code units): 16 lanes with three
    // units each, whose activation units the work-group keeps in LDS, leave
    // no lane idle where 64-lane rows idle a quarter of the wave.  Measured
    // on the Llama-3.2-3B shapes (K = 3072): LM head Q2 30.9 -> 27.3 us, Q3
    // 39.4 -> 35.3, Q4 43.5 -> 42.6; 8192 x 3072 Q2/Q3/Q4 5.9/6.5/6.2 ->
    // 5.3/5.5/5.8 us; 3072 x 3072 4.8/4.9/4.9 -> 4.3/4.2/4.3 us.
    if (!ls.multipass && ls.lpr == 64 && ls.xc == 1 && nu > 32 && nu <= 48 &&
        gemv_split_ok(16, 3))
        ls = {16, 3, false};
    const int el = override_or(OV_GEMV_LPR, 0), ex = override_or(OV_GEMV_XC, 0);
    if (el > 0 && ex > 0 && gemv_split_ok(el, ex)) ls = {el, ex, el * ex < nu};
    sh.lpr = ls.lpr;
    sh.xc = ls.xc;
    sh.multipass = ls.multipass;
    const int slots = 64 / sh.lpr;
    // Rows per slot per iteration: one when the row count alone fills the chip
    // with single-iteration waves; otherwise enough to keep ~128 bytes of
    // weights per lane in flight.
    // Rows per slot per iteration: one when the row count alone fills the
    // chip with single-iteration waves; otherwise two (the kernel keeps the
    // next iteration's loads in flight, so two rows per slot already hold
    // 2-4 units of weights per lane in flight).
    const int64_t waves_u1 = (n + slots - 1) / slots;
    int u = (waves_u1 > (int64_t)cus * 16 && sh.xc == 1) ? 2 : 1;
    while (u > 1 && !gemv_shape_supported(sh.lpr, sh.xc, u)) u /= 2;
    const int ev = override_or(OV_GEMV_U, 0);
    if (ev > 0 && gemv_shape_supported(sh.lpr, sh.xc, ev)) u = ev;
    sh.u = u;
    const int64_t batches = (n + (int64_t)slots * u - 1) / ((int64_t)slots * u);
    sh.work = batches;
    sh.cus = cus;
    // Matrices of up to 16 row batches per CU (the 3-15 MB projections) run
    // faster on a grid of two 4-wave work-groups per CU than at full
    // occupancy (measured 9-18 % on Llama-3.2-3B shapes: each wave streams
    // more batches through its pipelined loop); larger ones, the LM heads,
    // keep the occupancy-sized grid.
    const int wpc_default = batches <= (int64_t)16 * cus ? 8 : 0;
    // 64-lane rows with at least 16 batches per CU stage their row sums in
    // LDS (measured when K = 3072 rows still took 64 lanes, at Q4: the
    // 128256 x 3072 LM head 41.7 -> 41.4 us, 8192 x 3072 6.54 -> 6.15 us; Q2
    // 31.9 -> 30.6 and 6.35 -> 6.05 us; they now take 16 x 3 above);
    // with fewer batches per wave the staging round trip costs more than
    // the stores it moves (1024 x 3072: 3.9 -> 4.3 us), and 16-lane rows
    // lose by it too (151936 x 1024: 17.6 -> 18.2 us).
    // 16 x 3 rows stage too, from Q4 up: the staged loop's extra registers
    // (143 instead of 128 VGPRs: three waves per SIMD instead of four) cost
    // more than the stores it moves where the weights are fewest bytes per
    // instruction (the 128256 x 3072 LM head: Q4 43.1 -> 41.4 us staged, Q2
    // 27.3 -> 28.9, Q3 35.3 -> 35.6).
    const bool stageable = sh.lpr == 64 || (sh.lpr == 16 && sh.xc == 3 && bits >= 4);
    sh.staged = !sh.multipass && stageable && batches >= (int64_t)16 * cus;
    const int es = override_or(OV_GEMV_STAGED, -1);
    if (es >= 0) sh.staged = es == 1 && !sh.multipass && stageable;
    // Q4 rows of one unit per lane on at most 32 lanes (K up to 2048) build
    // their activation units after the first batch's weight loads, so the
    // two latencies overlap: 3072 x 1024 3.47 -> 3.21 us, 4096 x 1024 3.53
    // -> 3.34, 1024 x 2048 3.41 -> 3.16, 151936 x 1024 17.8 -> 17.1.  The
    // other shapes lost by it (8192 x 3072 5.62 -> 6.24, 1024 x 3072 3.86 ->
    // 4.17, 8192 x 2048 Q2 4.66 -> 4.96, 65536 x 1024 Q8 14.75 -> 15.38).
    const bool lateable = !sh.multipass && !sh.staged && bits == 4 && sh.lpr <= 32 && sh.xc == 1;
    sh.late = lateable;
    const int ol = override_or(OV_GEMV_LATE, -1);
    if (ol >= 0) sh.late = ol == 1 && lateable;
    sh.waves_per_cu = override_or(OV_GEMV_WAVES_PER_CU, wpc_default);
    // Reported grid: the cap assumes 16 resident waves per CU; the launch
    // uses the kernel's real occupancy.
    sh.grid = persistent_grid(sh.work, cus, sh.waves_per_cu > 0 ? sh.waves_per_cu / 4 : 4, 0);
    return sh;
}

// Batched GEMVs: one compiled shape (units per lane, rows per slot) for the
// launch, chosen from the largest K (at most 128 units per row) and the total
// row count; lanes per row are chosen per descriptor from its own K.
bool plan_batched(int64_t total_rows, int64_t kmax, int bits, int group, GemvShape* out) {
    GemvShape sh{};
    sh.unit = unit_codes(bits, group);
    const int nu = (int)(kmax / sh.unit);
    sh.xc = (nu + 63) / 64;
    if (sh.xc > 2) return false;
    sh.lpr = batched_lanes_per_row_host(nu, sh.xc);
    sh.multipass = false;
    // The row count decides, not the device, so prepared descriptors stay
    // valid on any GPU: big batches stream two rows per slot per iteration.
    // Two units per lane already double the registers; those keep one row.
    int u = (total_rows > (int64_t)16 * 4096 && sh.xc == 1) ? 2 : 1;
    const int ev = override_or(OV_BATCH_U, 0);
    if (ev > 0) u = ev;
    if (!batched_shape_supported(sh.xc, u)) u = 1;
    sh.u = u;
    *out = sh;
    return true;
}

constexpr int BATCHED_WAVES_PER_CU = 12;

// Row batches of one descriptor in a batched launch planned as sh.
int64_t batched_items(const GemvShape& sh, int64_t n, int64_t k) {
    const int lpr = batched_lanes_per_row_host((int)(k / sh.unit), sh.xc);
    const int64_t rows = (int64_t)(64 / lpr) * sh.u;
    return (n + rows - 1) / rows;
}

RowsShape plan_rows(int64_t rows_bound, int64_t n, int64_t k, int bits, int group, int cus,
                    int64_t n_seg_active) {
    RowsShape sh{};
    sh.unit = bits != 16 && group % 64 == 0 ? 64 : 32;
    const int nu = (int)(k / sh.unit);
    LaneSplit ls = choose_split(nu, 2, rows_split_ok);
    sh.lpr = ls.lpr;
    sh.xc = ls.xc;
    sh.multipass = ls.multipass;
    // Activation rows per MR-batch: what a segment is expected to hold
    // (rows spread over the active segments), at most 2 (1 with two units
    // per lane).
    const int64_t segs = n_seg_active > 0 ? n_seg_active : 1;
    const int64_t per_seg = (rows_bound + segs - 1) / segs;
    sh.mr = (per_seg <= 1 || sh.xc > 1) ? 1 : 2;
    const int em = override_or(OV_ROWS_MR, 0);
    if (em > 0 && rows_shape_supported(sh.lpr, sh.xc, em)) sh.mr = em;
    const int slots = 64 / sh.lpr;
    const int64_t rows_per_block = 4 * slots;
    const int64_t gx = (n + rows_per_block - 1) / rows_per_block;
    sh.grid_x = (int)(gx < INT_LIMIT ? gx : INT_LIMIT);
    // One work-group row per (segment, MR-row batch): at most
    // sum_e ceil(r_e / MR) <= (rows + (MR - 1) * segments) / MR of them.
    const int64_t pairs = (rows_bound + (int64_t)(sh.mr - 1) * segs + sh.mr - 1) / sh.mr;
    sh.pairs = (int)(pairs > 0 ? (pairs < INT_LIMIT ? pairs : INT_LIMIT) : 1);
    sh.grid_y = sh.pairs < 65535 ? sh.pairs : 65535;
    sh.cus = cus;
    // Little work (one token's experts: a handful of segments of one row) runs
    // faster on one 4-wave work-group per CU than at full occupancy
    // (measured ~20 % on the Qwen3-30B-A3B experts at one token: longer-lived
    // waves keep their pipelined loops busy); more work keeps the
    // occupancy-sized grid.
    const int64_t row_batches = (int64_t)sh.pairs * ((n + slots - 1) / slots);
    sh.waves_per_cu = override_or(OV_ROWS_WAVES_PER_CU, row_batches <= (int64_t)16 * cus ? 4 : 0);
    return sh;
}

// Tile height and K split.  Measured on the Llama-3.2-1B projections at
// m = 128 and 512: a work-group per CU (two for short splits) is the target;
// 64-row tiles win wherever they need no more work-groups than there are CUs
// (twice the waves per SIMD of the 128-row tile), except for long K with
// several 128-row tiles, where the 128-row tile's halved W traffic wins; a
// split shorter than four K steps costs more in partial sums than it gains.
// Splits up to this are added up inside the GEMM kernel by the last
// work-group of each tile (measured: 15.4 vs 18.7 us on 128 x 8192 x 2048);
// more splits go to a separate reduction kernel spread over the GPU (one
// work-group reading four or eight tiles' worth of partial sums measured
// 1-1.3 us slower than that kernel).
constexpr int GEMM_INKERNEL_REDUCE_MAX_SPLIT = 2;

// Split-K arrival counters: a fixed area at the start of the workspace, one
// int per output tile, the same for every shape so that the partial sums of
// one call (which follow it) never land on another call's counters.
constexpr size_t GEMM_COUNTER_BYTES = 4096;
constexpr int64_t GEMM_COUNTER_TILES = GEMM_COUNTER_BYTES / sizeof(int);

// n: output columns (the sum over the members of a grouped launch);
// tiles128: 128-column tiles (per member, summed); grouped launches keep
// 128-column tiles and split K only where the kernel reduces the split
// itself (32/64-row tiles, counters for every tile).
// Workspace for a split plan: the arrival counters, then the partial sums
// (their byte offsets must stay below 2^32).  Shrinks the split to what the
// caller's workspace holds.
int fit_split(int split, int64_t m, int64_t n, size_t ws_bytes, size_t* ws_need) {
    const size_t per_split = (size_t)m * n * sizeof(float);
    const size_t cnt_bytes = GEMM_COUNTER_BYTES;
    if (per_split && split > 1 && per_split * split > 0xFFFFFFFFull) split = (int)(0xFFFFFFFFull / per_split);
    if (ws_need) *ws_need = split > 1 ? cnt_bytes + per_split * split : 0;
    if (split > 1 && ws_bytes < cnt_bytes + per_split * split) {
        split = (per_split && ws_bytes > cnt_bytes) ? (int)((ws_bytes - cnt_bytes) / per_split) : 1;
        if (split < 2) split = 1;
    }
    return split;
}

// The LDS-dequantizing kernel (gemm_wl.hip).  Its 256 x 256 tiles read the
// fewest LDS bytes per matrix instruction (the limit of both kernels once
// the dequantization is off the matrix waves): measured 76.3 vs 82.8 us on
// the 8192 x 2048 projections at 2048 tokens.  It takes the shapes whose
// 256 x 256 grid alone fills the CUs; the override QMM_GEMM_KERNEL = 1
// forces it elsewhere (tiles 256 x 128 above 128 rows, else 128 x 128,
// unless QMM_GEMM_TILE_M / _N say otherwise).
bool wl_fills(int64_t m, int64_t n, int cus) { return (m + 255) / 256 * ((n + 255) / 256) >= cus; }

// member_n / members: a grouped launch's column counts; its column tiles are
// counted per member (each member's last tile may be partial).
GemmShape plan_gemm_wl(int64_t m, int64_t n, int64_t k, int cus, size_t ws_bytes, size_t* ws_need,
                       const int64_t* member_n = nullptr, int members = 0, int tile_n = 256) {
    GemmShape sh{};
    sh.kernel = 1;
    const bool forced = override_or(OV_GEMM_KERNEL, 0) == 1;
    sh.tile_m = forced ? (m > 128 ? 256 : 128) : 256;
    sh.tile_n = forced ? 128 : tile_n;
    const int etm = override_or(OV_GEMM_TILE_M, 0);
    if (etm == 128 || etm == 256) sh.tile_m = etm;
    const int etn = override_or(OV_GEMM_TILE_N, 0);
    if (etn == 128 || etn == 256) sh.tile_n = etn;
    sh.grid_m = (int)((m + sh.tile_m - 1) / sh.tile_m);
    if (members) {
        int64_t t = 0;
        for (int j = 0; j < members; ++j) t += (member_n[j] + sh.tile_n - 1) / sh.tile_n;
        sh.grid_n = (int)t;
    } else {
        sh.grid_n = (int)((n + sh.tile_n - 1) / sh.tile_n);
    }
    const int k_tiles = (int)((k + gemm_wl_step_codes(sh.tile_n) - 1) / gemm_wl_step_codes(sh.tile_n));
    const int64_t tiles = (int64_t)sh.grid_m * sh.grid_n;
    int split = 1;
    if (tiles < cus) {
        split = (int)((cus + tiles - 1) / tiles);
        const int by_k = k_tiles / 2 > 1 ? k_tiles / 2 : 1;
        if (split > by_k) split = by_k;
    }
    const int es = override_or(OV_GEMM_SPLIT, 0);
    if (es > 0) split = es < k_tiles ? es : k_tiles;
    if (split > 16) split = 16;
    // A grouped launch reduces its splits in the kernel: one counter per tile.
    if (members && tiles > GEMM_COUNTER_TILES) split = 1;
    split = fit_split(split, m, n, ws_bytes, ws_need);
    sh.k_tiles_per_split = (k_tiles + split - 1) / split;
    sh.split = (k_tiles + sh.k_tiles_per_split - 1) / sh.k_tiles_per_split;
    sh.wide_scales = false;
    // Tile order: an XCD's consecutive tiles share X rows (column tile
    // fastest) or W columns (row tile fastest); take the order that moves
    // fewer bytes into the XCDs: X once plus W once per row tile, or W once
    // plus X once per column tile.
    const double xb = 2.0 * (double)m * (double)k, wb = 0.5 * (double)n * (double)k;
    const bool col_fastest = xb + sh.grid_m * wb <= wb + sh.grid_n * xb;
    const int eo = override_or(OV_GEMM_ORDER, 0);
    sh.n_fast = eo == 1 ? true : eo == 2 ? false : col_fastest;
    return sh;
}

GemmShape plan_gemm_impl(int64_t m, int64_t n, int64_t tiles128, bool grouped, int64_t k, int group, int bits, int cus,
                         size_t ws_bytes, size_t* ws_need) {
    const int ek = override_or(OV_GEMM_KERNEL, 0);
    if (!grouped && (ek == 1 || (ek != 2 && m > 128 && wl_fills(m, n, cus))))
        return plan_gemm_wl(m, n, k, cus, ws_bytes, ws_need);
    GemmShape sh{};
    const int k_tiles = (int)((k + GEMM_BK - 1) / GEMM_BK);
    const int64_t grid_n = tiles128;
    sh.tile_m = m <= 32 ? 32 : m <= 64 ? 64 : 128;
    if (sh.tile_m == 128) {
        const int64_t tiles64 = (m + 63) / 64 * grid_n;
        const bool long_k = k_tiles >= 64 && m > 128;
        if (tiles64 <= cus && !long_k) sh.tile_m = 64;
    }
    // 32-row tiles where 64-row ones would split a short K: twice the tiles
    // for the same split count, or no split at all (128 tokens, 2048 x 2048:
    // 8.3 against 9.2 us; q|k|v grouped at 512 tokens: 19.5 against 22.5).
    // A long K keeps 64-row tiles (W is read once per row tile), and so do
    // fp16 weights, four times the bytes to re-read (2048 x 2048 at 512
    // tokens: 25.1 against 18.0 us).
    if (sh.tile_m == 64 && m > 64 && bits != 16 && (m + 63) / 64 * grid_n < cus && k_tiles < 64) sh.tile_m = 32;
    const int et = override_or(OV_GEMM_TILE_M, 0);
    if (et == 32 || et == 64 || et == 128) sh.tile_m = et;
    // 128 x 256 tiles (eight waves along N, whole steps each) halve the X
    // bytes per flop; they pay off where their grid alone fills the CUs
    // (measured: 12 % on 8192 x 2048 at m = 2048, a loss wherever they would
    // need a K split).
    sh.tile_n = (!grouped && sh.tile_m == 128 && (m + 127) / 128 * ((n + 255) / 256) >= cus) ? 256 : 128;
    const int etn = override_or(OV_GEMM_TILE_N, 0);
    if (!grouped && (etn == 128 || etn == 256) && sh.tile_m >= 64) sh.tile_n = etn;
    sh.grid_m = (int)((m + sh.tile_m - 1) / sh.tile_m);
    sh.grid_n = grouped ? (int)tiles128 : (int)((n + sh.tile_n - 1) / sh.tile_n);
    const int64_t tiles = (int64_t)sh.grid_m * sh.grid_n;
    int split = 1;
    if (tiles < cus) {
        split = (int)((cus + tiles - 1) / tiles);
        const int by_k = k_tiles / 4 > 1 ? k_tiles / 4 : 1;
        if (split > by_k) split = by_k;
        if (split > 16) split = 16;
    }
    const int es = override_or(OV_GEMM_SPLIT, 0);
    if (es > 0) split = es < k_tiles ? es : k_tiles;
    if (split > 16) split = 16;  // the reduction handles at most 16 splits
    if (grouped && (sh.tile_m > 64 || tiles > GEMM_COUNTER_TILES)) split = 1;
    split = fit_split(split, m, n, ws_bytes, ws_need);
    sh.k_tiles_per_split = (k_tiles + split - 1) / split;
    // Wide scale loads need splits that start at multiples of four steps.
    const bool wide = group == 64 && GEMM_BK == 128 && k % 512 == 0 && override_or(OV_GEMM_WIDE_SCALES, 1) != 0;
    if (wide && split > 1) sh.k_tiles_per_split = (sh.k_tiles_per_split + 3) / 4 * 4;
    sh.split = (k_tiles + sh.k_tiles_per_split - 1) / sh.k_tiles_per_split;
    sh.wide_scales = wide;
    // The rounding above can leave fewer splits than were fitted: the
    // workspace is what the final split count uses.
    if (ws_need) *ws_need = sh.split > 1 ? GEMM_COUNTER_BYTES + (size_t)m * n * sizeof(float) * sh.split : 0;
    // Tile order (see gemm_kernel): column tiles fastest from 16 row tiles
    // on, unless there are more column tiles than row tiles (8192 x 2048 at
    // 2048 tokens: +1 % that way).
    const int eo = override_or(OV_GEMM_ORDER, 0);
    sh.n_fast = eo == 1 ? true : eo == 2 ? false : (sh.grid_m >= 16 && sh.grid_n <= sh.grid_m);
    return sh;
}

// Splits summed inside the GEMM kernel (arrival counters in the workspace):
// two-way splits of the tiles that have that reduction.
bool reduces_in_kernel(const GemmShape& sh) {
    if (sh.split < 2 || sh.split > GEMM_INKERNEL_REDUCE_MAX_SPLIT) return false;
    if ((int64_t)sh.grid_m * sh.grid_n > GEMM_COUNTER_TILES) return false;
    return sh.kernel == 1 || (sh.tile_m <= 64 && sh.tile_n == 128);
}

GemmShape plan_gemm(int64_t m, int64_t n, int64_t k, int group, int bits, int cus, size_t ws_bytes,
                    size_t* ws_need) {
    return plan_gemm_impl(m, n, (n + 127) / 128, false, k, group, bits, cus, ws_bytes, ws_need);
}

// m rows at or below this go to the multi-row GEMV kernel instead of MFMA.
constexpr int64_t ROWS_KERNEL_MAX_M = 2;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

qmm_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(QMM_ERR_DEVICE, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int qmm_abi_version(void) { return QMM_ABI_VERSION; }

const char* qmm_last_error(void) { return g_err; }

const char* qmm_status_string(qmm_status s) {
    switch (s) {
        case QMM_OK: return "QMM_OK";
        case QMM_ERR_INVALID_ARGUMENT: return "QMM_ERR_INVALID_ARGUMENT";
        case QMM_ERR_UNSUPPORTED: return "QMM_ERR_UNSUPPORTED";
        case QMM_ERR_MISALIGNED: return "QMM_ERR_MISALIGNED";
        case QMM_ERR_DEVICE: return "QMM_ERR_DEVICE";
        default: return "QMM_ERR_UNKNOWN";
    }
}

qmm_status qmm_gemv(const void* w_packed, const void* scales, const void* mins, const void* x,
                    float* y, int64_t n, int64_t k, int bits, int group_size, void* stream) {
    qmm_status st = check_format(n, k, bits, group_size);
    if (st != QMM_OK) return st;
    if (n == 0) return ok();
    if ((st = check_weight_ptrs(w_packed, scales, mins, bits)) != QMM_OK) return st;
    if (!x || !y) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL x or y");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(QMM_ERR_MISALIGNED, "x or y not 16-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    const GemvShape sh = plan_gemv(n, k, bits, group_size, cus);
    GemvArgs a{static_cast<const uint32_t*>(w_packed), static_cast<const uint16_t*>(scales),
               static_cast<const uint16_t*>(mins), static_cast<const uint16_t*>(x), y, (int)n, (int)k,
               group_size, bits};
    return launched(launch_gemv(a, sh, as_stream(stream)), "qmm_gemv");
}

qmm_status qmm_gemv_residual(const void* w_packed, const void* scales, const void* mins, const void* x,
                             const float* residual, float* y, int64_t n, int64_t k, int bits,
                             int group_size, void* stream) {
    qmm_status st = check_format(n, k, bits, group_size);
    if (st != QMM_OK) return st;
    if (n == 0) return ok();
    if ((st = check_weight_ptrs(w_packed, scales, mins, bits)) != QMM_OK) return st;
    if (!x || !y || !residual) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL x, residual or y");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(QMM_ERR_MISALIGNED, "x or y not 16-byte aligned");
    if (!aligned(residual, 4)) return fail(QMM_ERR_MISALIGNED, "residual not 4-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    const GemvShape sh = plan_gemv(n, k, bits, group_size, cus);
    GemvArgs a{static_cast<const uint32_t*>(w_packed), static_cast<const uint16_t*>(scales),
               static_cast<const uint16_t*>(mins), static_cast<const uint16_t*>(x), y, (int)n, (int)k,
               group_size, bits, residual};
    return launched(launch_gemv(a, sh, as_stream(stream)), "qmm_gemv_residual");
}

qmm_status qmm_gemv_swiglu(const void* gate_w, const void* gate_scales, const void* gate_mins,
                           const void* up_w, const void* up_scales, const void* up_mins, const void* x,
                           float* h, int64_t n, int64_t k, int bits, int group_size, void* stream) {
    qmm_status st = check_format(n, k, bits, group_size);
    if (st != QMM_OK) return st;
    if (n == 0) return ok();
    if ((st = check_weight_ptrs(gate_w, gate_scales, gate_mins, bits)) != QMM_OK) return st;
    if ((st = check_weight_ptrs(up_w, up_scales, up_mins, bits)) != QMM_OK) return st;
    if (!x || !h) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL x or h");
    if (!aligned(x, 16) || !aligned(h, 16)) return fail(QMM_ERR_MISALIGNED, "x or h not 16-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    GemvShape sh = plan_gemv(n, k, bits, group_size, cus);
    if (sh.multipass || !glu_shape_supported(sh.lpr, sh.xc))
        return fail(QMM_ERR_UNSUPPORTED, "k=%lld needs more than one pass of the fused gate/up kernel",
                    (long long)k);
    sh.u = 1;
    sh.work = (n + 64 / sh.lpr - 1) / (64 / sh.lpr);
    GluArgs a{static_cast<const uint32_t*>(gate_w), static_cast<const uint16_t*>(gate_scales),
              static_cast<const uint16_t*>(gate_mins), static_cast<const uint32_t*>(up_w),
              static_cast<const uint16_t*>(up_scales), static_cast<const uint16_t*>(up_mins),
              static_cast<const uint16_t*>(x), h, (int)n, (int)k, group_size, bits};
    return launched(launch_glu(a, sh, as_stream(stream)), "qmm_gemv_swiglu");
}

size_t qmm_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int bits, int group_size) {
    if (check_format(n, k, bits, group_size) != QMM_OK || m <= ROWS_KERNEL_MAX_M || n == 0) return 0;
    int cus = 0;
    if (device_cus(&cus) != QMM_OK) cus = 256;
    size_t need = 0;
    (void)plan_gemm(m, n, k, group_size, bits, cus, (size_t)-1, &need);
    return need;
}

}  // extern "C"

namespace {

// ---- scratch of qmm_gemm_noalloc ---------------------------------------------
// K-split partial sums and arrival counters of the allocation-free GEMM: one
// array per GPU, part of the library's code object, held until the process
// ends.  In host code `scratch` names a host-side stand-in, not device
// memory: each device's own copy is found once with hipGetSymbolAddress
// (with that device current) and only that address is passed on.
static __device__ __align__(256) unsigned char scratch[QMM_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_addr[MAX_DEVICES];
std::mutex g_scratch_mutex;

qmm_status device_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(QMM_ERR_DEVICE, "no HIP device available");
    }
    if (dev < 0 || dev >= MAX_DEVICES) return fail(QMM_ERR_UNSUPPORTED, "device %d beyond %d", dev, MAX_DEVICES);
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                (void)hipGetLastError();
                return fail(QMM_ERR_DEVICE, "scratch address on device %d: %s", dev, hipGetErrorString(e));
            }
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return QMM_OK;
}

// Zero `count` ints (a kernel rather than a memset node, so the call stays
// safe to capture into a graph).
__global__ void clear_ints_kernel(int* __restrict__ p, int count) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

// qmm_gemm and qmm_gemm_f16out.  fp16 output always takes the MFMA kernel
// (its epilogue does the rounding); fp32 output routes m <= 2 to the GEMV
// kernels.
qmm_status gemm_common(const void* w_packed, const void* scales, const void* mins, const void* x,
                       void* y, int64_t m, int64_t n, int64_t k, int bits, int group_size,
                       void* workspace, size_t workspace_bytes, void* stream, bool out16,
                       bool noalloc = false) {
    qmm_status st = check_format(n, k, bits, group_size);
    if (st != QMM_OK) return st;
    if (m < 0) return fail(QMM_ERR_INVALID_ARGUMENT, "m=%lld is negative", (long long)m);
    if (m > INT_LIMIT || m * n > ((int64_t)1 << 40))
        return fail(QMM_ERR_INVALID_ARGUMENT, "m too large");
    if (m == 0 || n == 0) return ok();
    if ((st = check_activation_bytes(m, k)) != QMM_OK) return st;
    if ((st = check_output_bytes(m, n)) != QMM_OK) return st;
    if ((st = check_weight_ptrs(w_packed, scales, mins, bits)) != QMM_OK) return st;
    if (!x || !y) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL x or y");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(QMM_ERR_MISALIGNED, "x or y not 16-byte aligned");
    if (workspace_bytes && !workspace)
        return fail(QMM_ERR_INVALID_ARGUMENT, "workspace_bytes > 0 with a NULL workspace");
    if (workspace && !aligned(workspace, 16)) return fail(QMM_ERR_MISALIGNED, "workspace not 16-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    const uint32_t* w = static_cast<const uint32_t*>(w_packed);
    const uint16_t* s = static_cast<const uint16_t*>(scales);
    const uint16_t* mn = static_cast<const uint16_t*>(mins);
    const uint16_t* xx = static_cast<const uint16_t*>(x);
    float* yf = static_cast<float*>(y);
    if (!out16 && m == 1) {
        const GemvShape sh = plan_gemv(n, k, bits, group_size, cus);
        GemvArgs a{w, s, mn, xx, yf, (int)n, (int)k, group_size, bits};
        return launched(launch_gemv(a, sh, as_stream(stream)), "qmm_gemm (gemv)");
    }
    if (!out16 && m <= ROWS_KERNEL_MAX_M) {
        const RowsShape sh = plan_rows(m, n, k, bits, group_size, cus, 1);
        RowsArgs a{w, s, mn, xx, nullptr, (int)m, nullptr, 1, (int)m, yf, (int)n, (int)k, group_size, bits};
        return launched(launch_rows(a, sh, as_stream(stream)), "qmm_gemm (rows)");
    }
    if (noalloc) {
        // The plan qmm_gemm takes with its preferred workspace, on the
        // library's own scratch array.
        size_t need = 0;
        (void)plan_gemm(m, n, k, group_size, bits, cus, (size_t)-1, &need);
        if (need > (size_t)QMM_NOALLOC_SCRATCH_BYTES)
            return fail(QMM_ERR_UNSUPPORTED,
                        "m=%lld n=%lld k=%lld needs %zu bytes of scratch, more than the %zu this entry point holds",
                        (long long)m, (long long)n, (long long)k, need, (size_t)QMM_NOALLOC_SCRATCH_BYTES);
        if ((st = device_scratch(&workspace)) != QMM_OK) return st;
        workspace_bytes = need;
    }
    const GemmShape sh = plan_gemm(m, n, k, group_size, bits, cus, workspace ? workspace_bytes : 0, nullptr);
    float* partial = nullptr;
    int* counters = nullptr;
    if (sh.split > 1) {
        partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + GEMM_COUNTER_BYTES);
        if (reduces_in_kernel(sh)) counters = static_cast<int*>(workspace);
    }
    if (noalloc && counters) {
        // The shared array keeps whatever the last call left: the arrival
        // counters this launch uses start from zero.
        const int used = sh.grid_m * sh.grid_n;
        hipLaunchKernelGGL(clear_ints_kernel, dim3((used + 255) / 256), dim3(256), 0, as_stream(stream), counters,
                           used);
        if (hipError_t e = hipGetLastError(); e != hipSuccess)
            return fail(QMM_ERR_DEVICE, "qmm_gemm_noalloc: counter reset failed: %s", hipGetErrorString(e));
    }
    GemmArgs a{w, s, mn, xx, yf, partial, counters, (int)m, (int)n, (int)k, group_size, bits, out16 ? 1 : 0};
    return launched(launch_gemm(a, sh, as_stream(stream)),
                    noalloc ? "qmm_gemm_noalloc" : out16 ? "qmm_gemm_f16out" : "qmm_gemm");
}

}  // namespace

extern "C" {

// Members of a grouped GEMM, checked, with zero-column members dropped.
static qmm_status check_group(const qmm_gemm_member* members, int count, int64_t m, int64_t k, int bits,
                              int group_size, int64_t* ns, int* kept, int64_t* n_sum, int64_t* tiles128,
                              bool pointers = true) {
    if (count < 1 || count > GEMM_GROUP_MAX)
        return fail(QMM_ERR_INVALID_ARGUMENT, "count=%d outside 1..%d", count, GEMM_GROUP_MAX);
    if (!members) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL members");
    *kept = 0;
    *n_sum = 0;
    *tiles128 = 0;
    char why[sizeof g_err];
    for (int i = 0; i < count; ++i) {
        const qmm_gemm_member& g = members[i];
        qmm_status st = check_format(g.n, k, bits, group_size);
        const bool live = g.n > 0 && m > 0;
        if (st == QMM_OK && live) st = check_output_bytes(m, g.n);
        if (st == QMM_OK && live && pointers) st = check_weight_ptrs(g.w_packed, g.scales, g.mins, bits);
        if (st == QMM_OK && live && pointers && !g.y) st = fail(QMM_ERR_INVALID_ARGUMENT, "NULL y");
        if (st == QMM_OK && live && pointers && !aligned(g.y, 16))
            st = fail(QMM_ERR_MISALIGNED, "y not 16-byte aligned");
        if (st != QMM_OK) {
            memcpy(why, g_err, sizeof why);
            return fail(st, "member %d: %s", i, why);
        }
        if (g.n == 0) continue;
        ns[(*kept)++] = i;
        *n_sum += g.n;
        *tiles128 += (g.n + 127) / 128;
    }
    if (*n_sum > INT_LIMIT) return fail(QMM_ERR_INVALID_ARGUMENT, "total n above 2^31-1");
    return QMM_OK;
}

// Column tiles of a grouped launch at tile width tn (per member).
static int64_t grouped_tiles(const qmm_gemm_member* members, const int64_t* idx, int kept, int64_t tn) {
    int64_t t = 0;
    for (int j = 0; j < kept; ++j) t += (members[idx[j]].n + tn - 1) / tn;
    return t;
}

// Whether one grouped launch of the LDS-dequantizing kernel (256-row tiles)
// fills the CUs without a K split: then it beats both separate launches and
// the register kernel's grouped launch (gate|up at 512 tokens: 46.3 us
// against 51.7 for two launches; q|k|v, whose grids stay below the CU
// count, lose 2-3x on it through their K splits).
static bool grouped_wl_fills(const qmm_gemm_member* members, const int64_t* idx, int kept, int64_t m, int cus) {
    if (m <= 128) return false;
    return (m + 255) / 256 * grouped_tiles(members, idx, kept, 128) >= cus;
}

// A grouped launch pays where the members underfill the GPU on their own
// (q|k|v, and gate|up at 128 tokens: 11.5 vs 27.8 us and 17.9 vs 28.0 us);
// where every member's own tile grid already fills it, separate launches
// keep the best tile shape per member (gate|up at 2048 tokens: 159 us
// separate against 205 grouped).
static bool members_fill_alone(const qmm_gemm_member* members, const int64_t* idx, int kept, int64_t m,
                               int64_t k, int group_size, int bits, int cus) {
    if (override_or(OV_GEMM_GROUPED, 0) == 1) return false;  // always one launch (for measurements)
    bool all_wl = true;
    for (int j = 0; j < kept; ++j) {
        const GemmShape sh = plan_gemm(m, members[idx[j]].n, k, group_size, bits, cus, 0, nullptr);
        // A member fills the GPU alone with tiles of at least 64 rows (32-row
        // tiles fill it only by re-reading W twice as often: gate|up at 128
        // tokens take 28.3 us as two such launches, 18.8 as one grouped).
        const int64_t tm = sh.kernel == 1 || sh.tile_m >= 64 ? sh.tile_m : 64;
        if ((m + tm - 1) / tm * sh.grid_n < cus) return false;
        all_wl = all_wl && sh.kernel == 1;
    }
    // Members that fill the GPU only with the register kernel's tiles go
    // into one launch of the LDS kernel where that launch fills it too.
    if (!all_wl && override_or(OV_GEMM_KERNEL, 0) != 2 && grouped_wl_fills(members, idx, kept, m, cus))
        return false;
    return true;
}

// The plan of one grouped launch: the LDS-dequantizing kernel where
// QMM_GEMM_KERNEL = 1 asks for it or where its grouped grid fills the CUs
// (256 x 256 tiles if those fill them, else 256 x 128), else the register-
// dequantizing kernel's 128-column tiles.
static GemmShape plan_grouped(const qmm_gemm_member* members, const int64_t* idx, int kept, int64_t m,
                              int64_t k, int group_size, int bits, int cus, int64_t n_sum, int64_t tiles128,
                              size_t ws_bytes, size_t* ws_need) {
    const int ek = override_or(OV_GEMM_KERNEL, 0);
    if (ek == 1 || (ek != 2 && grouped_wl_fills(members, idx, kept, m, cus))) {
        int64_t ns[GEMM_GROUP_MAX];
        for (int j = 0; j < kept; ++j) ns[j] = members[idx[j]].n;
        const bool wide = (m + 255) / 256 * grouped_tiles(members, idx, kept, 256) >= cus;
        return plan_gemm_wl(m, n_sum, k, cus, ws_bytes, ws_need, ns, kept, wide ? 256 : 128);
    }
    return plan_gemm_impl(m, n_sum, tiles128, true, k, group_size, bits, cus, ws_bytes, ws_need);
}

size_t qmm_gemm_grouped_workspace_bytes(const qmm_gemm_member* members, int count, int64_t m, int64_t k,
                                        int bits, int group_size) {
    int64_t idx[GEMM_GROUP_MAX];
    int kept = 0;
    int64_t n_sum = 0, tiles128 = 0;
    if (m <= 0 ||
        check_group(members, count, m, k, bits, group_size, idx, &kept, &n_sum, &tiles128, false) != QMM_OK ||
        kept == 0)
        return 0;
    int cus = 0;
    if (device_cus(&cus) != QMM_OK) cus = 256;
    size_t need = 0;
    if (members_fill_alone(members, idx, kept, m, k, group_size, bits, cus)) {
        for (int j = 0; j < kept; ++j) {
            size_t one = 0;
            (void)plan_gemm(m, members[idx[j]].n, k, group_size, bits, cus, (size_t)-1, &one);
            if (one > need) need = one;
        }
        return need;
    }
    (void)plan_grouped(members, idx, kept, m, k, group_size, bits, cus, n_sum, tiles128, (size_t)-1, &need);
    return need;
}

qmm_status qmm_gemm_grouped(const qmm_gemm_member* members, int count, const void* x, int64_t m, int64_t k,
                            int bits, int group_size, void* workspace, size_t workspace_bytes, void* stream) {
    if (m < 0) return fail(QMM_ERR_INVALID_ARGUMENT, "m=%lld is negative", (long long)m);
    if (m > INT_LIMIT) return fail(QMM_ERR_INVALID_ARGUMENT, "m too large");
    int64_t idx[GEMM_GROUP_MAX];
    int kept = 0;
    int64_t n_sum = 0, tiles128 = 0;
    qmm_status st = check_group(members, count, m, k, bits, group_size, idx, &kept, &n_sum, &tiles128);
    if (st != QMM_OK) return st;
    if (m == 0 || kept == 0) return ok();
    if ((st = check_activation_bytes(m, k)) != QMM_OK) return st;
    if (!x) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL x");
    if (!aligned(x, 16)) return fail(QMM_ERR_MISALIGNED, "x not 16-byte aligned");
    if (workspace_bytes && !workspace)
        return fail(QMM_ERR_INVALID_ARGUMENT, "workspace_bytes > 0 with a NULL workspace");
    if (workspace && !aligned(workspace, 16)) return fail(QMM_ERR_MISALIGNED, "workspace not 16-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    if (members_fill_alone(members, idx, kept, m, k, group_size, bits, cus)) {
        for (int j = 0; j < kept; ++j) {
            const qmm_gemm_member& mb = members[idx[j]];
            if ((st = gemm_common(mb.w_packed, mb.scales, mb.mins, x, mb.y, m, mb.n, k, bits, group_size,
                                  workspace, workspace_bytes, stream, false)) != QMM_OK)
                return st;
        }
        return ok();
    }
    const GemmShape sh = plan_grouped(members, idx, kept, m, k, group_size, bits, cus, n_sum, tiles128,
                                      workspace ? workspace_bytes : 0, nullptr);
    const int tile_n = sh.kernel == 1 ? sh.tile_n : 128;
    GemmGroupArgs g{};
    g.count = kept;
    int tile = 0, col = 0;
    for (int j = 0; j < kept; ++j) {
        const qmm_gemm_member& mb = members[idx[j]];
        g.w[j] = static_cast<const uint32_t*>(mb.w_packed);
        g.s[j] = static_cast<const uint16_t*>(mb.scales);
        g.m[j] = static_cast<const uint16_t*>(mb.mins);
        g.y[j] = mb.y;
        g.n[j] = (int)mb.n;
        g.col0[j] = col;
        g.tile0[j] = tile;
        col += (int)mb.n;
        tile += (int)((mb.n + tile_n - 1) / tile_n);
    }
    for (int j = kept; j <= GEMM_GROUP_MAX; ++j) g.tile0[j] = tile;
    float* partial = nullptr;
    int* counters = nullptr;
    if (sh.split > 1) {
        counters = static_cast<int*>(workspace);
        partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + GEMM_COUNTER_BYTES);
    }
    GemmArgs a{g.w[0], g.s[0], g.m[0], static_cast<const uint16_t*>(x), g.y[0], partial, counters, (int)m,
               (int)n_sum, (int)k, group_size, bits, 0};
    a.grp = &g;
    return launched(launch_gemm(a, sh, as_stream(stream)), "qmm_gemm_grouped");
}

qmm_status qmm_gemm(const void* w_packed, const void* scales, const void* mins, const void* x,
                    float* y, int64_t m, int64_t n, int64_t k, int bits, int group_size,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_common(w_packed, scales, mins, x, y, m, n, k, bits, group_size, workspace,
                       workspace_bytes, stream, false);
}

qmm_status qmm_gemm_f16out(const void* w_packed, const void* scales, const void* mins, const void* x,
                           void* y, int64_t m, int64_t n, int64_t k, int bits, int group_size,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return gemm_common(w_packed, scales, mins, x, y, m, n, k, bits, group_size, workspace,
                       workspace_bytes, stream, true);
}

qmm_status qmm_gemm_noalloc(const void* w_packed, const void* scales, const void* mins, const void* x,
                            float* y, int64_t m, int64_t n, int64_t k, int bits, int group_size,
                            void* stream) {
    return gemm_common(w_packed, scales, mins, x, y, m, n, k, bits, group_size, nullptr, 0, stream, false,
                       true);
}

qmm_status qmm_set_override(const char* name, int value) {
    if (!name) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL override name");
    for (int i = 0; i < OV_COUNT; ++i)
        if (strcmp(name, OVERRIDE_NAMES[i]) == 0) {
            g_override[i].store(value < 0 ? -1 : value, std::memory_order_relaxed);
            return ok();
        }
    return fail(QMM_ERR_INVALID_ARGUMENT, "unknown override %s", name);
}

}  // extern "C"

namespace {

// qmm_moe_gemm, and qmm_moe_swiglu when up_w is given (y = silu(W x) * (Wup x)).
qmm_status moe_common(const void* w_packed, const void* scales, const void* mins, const void* up_w,
                      const void* up_s, const void* up_m, const void* x, const int32_t* x_rows,
                      int64_t x_rows_count, const int32_t* expert_offsets, float* y, int64_t p_rows,
                      int64_t n_experts, int64_t n, int64_t k, int bits, int group_size, void* stream,
                      bool glu, const int32_t* pair_token = nullptr, const float* pair_weight = nullptr,
                      int64_t n_tokens = 0) {
    const bool combine = pair_token != nullptr || pair_weight != nullptr;
    qmm_status st = check_format(n, k, bits, group_size);
    if (st != QMM_OK) return st;
    if (p_rows < 0 || n_experts < 0 || x_rows_count < 0)
        return fail(QMM_ERR_INVALID_ARGUMENT, "negative p_rows, n_experts or x_rows_count");
    if (p_rows > INT_LIMIT || n_experts > INT_LIMIT || x_rows_count > INT_LIMIT)
        return fail(QMM_ERR_INVALID_ARGUMENT, "p_rows, n_experts or x_rows_count above 2^31-1");
    if (combine && (n_tokens < 0 || n_tokens > INT_LIMIT))
        return fail(QMM_ERR_INVALID_ARGUMENT, "n_tokens=%lld out of range", (long long)n_tokens);
    if (p_rows == 0 || n == 0 || n_experts == 0 || (combine && n_tokens == 0)) return ok();
    if ((st = check_activation_bytes(x_rows ? x_rows_count : p_rows, k)) != QMM_OK) return st;
    if ((st = check_output_bytes(combine ? n_tokens : p_rows, n)) != QMM_OK) return st;
    if (combine && (!pair_token || !pair_weight))
        return fail(QMM_ERR_INVALID_ARGUMENT, "NULL pair_token or pair_weight");
    if (combine && (!aligned(pair_token, 4) || !aligned(pair_weight, 4)))
        return fail(QMM_ERR_MISALIGNED, "pair_token or pair_weight not 4-byte aligned");
    if ((st = check_weight_ptrs(w_packed, scales, mins, bits)) != QMM_OK) return st;
    if (glu && (st = check_weight_ptrs(up_w, up_s, up_m, bits)) != QMM_OK) return st;
    if (!x || !y || !expert_offsets) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL x, y or expert_offsets");
    if (!x_rows && x_rows_count < p_rows)
        return fail(QMM_ERR_INVALID_ARGUMENT, "x_rows is NULL and x has fewer than p_rows rows");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(QMM_ERR_MISALIGNED, "x or y not 16-byte aligned");
    if (!aligned(expert_offsets, 4) || (x_rows && !aligned(x_rows, 4)))
        return fail(QMM_ERR_MISALIGNED, "index arrays not 4-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    const int64_t active = n_experts < p_rows ? n_experts : p_rows;
    const RowsShape sh = plan_rows(p_rows, n, k, bits, group_size, cus, active);
    if (glu && sh.multipass)
        return fail(QMM_ERR_UNSUPPORTED, "k=%lld needs more than one pass of the fused gate/up kernel",
                    (long long)k);
    RowsArgs a{static_cast<const uint32_t*>(w_packed), static_cast<const uint16_t*>(scales),
               static_cast<const uint16_t*>(mins), static_cast<const uint16_t*>(x), x_rows,
               (int)(x_rows ? x_rows_count : p_rows), expert_offsets, (int)n_experts, (int)p_rows, y, (int)n, (int)k,
               group_size, bits};
    if (combine) {
        a.pair_token = pair_token;
        a.pair_weight = pair_weight;
        a.n_tokens = (int)n_tokens;
    }
    if (glu) {
        a.w2 = static_cast<const uint32_t*>(up_w);
        a.s2 = static_cast<const uint16_t*>(up_s);
        a.m2 = static_cast<const uint16_t*>(up_m);
    }
    return launched(launch_rows(a, sh, as_stream(stream)),
                    glu ? "qmm_moe_swiglu" : combine ? "qmm_moe_combine" : "qmm_moe_gemm");
}

}  // namespace

extern "C" {

qmm_status qmm_moe_gemm(const void* w_packed, const void* scales, const void* mins, const void* x,
                        const int32_t* x_rows, int64_t x_rows_count, const int32_t* expert_offsets,
                        float* y, int64_t p_rows, int64_t n_experts, int64_t n, int64_t k, int bits,
                        int group_size, void* stream) {
    return moe_common(w_packed, scales, mins, nullptr, nullptr, nullptr, x, x_rows, x_rows_count,
                      expert_offsets, y, p_rows, n_experts, n, k, bits, group_size, stream, false);
}

qmm_status qmm_moe_combine(const void* w_packed, const void* scales, const void* mins, const void* x,
                           const int32_t* x_rows, int64_t x_rows_count, const int32_t* expert_offsets,
                           const int32_t* pair_token, const float* pair_weight, float* y, int64_t n_tokens,
                           int64_t p_rows, int64_t n_experts, int64_t n, int64_t k, int bits,
                           int group_size, void* stream) {
    if (!pair_token || !pair_weight) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL pair_token or pair_weight");
    return moe_common(w_packed, scales, mins, nullptr, nullptr, nullptr, x, x_rows, x_rows_count,
                      expert_offsets, y, p_rows, n_experts, n, k, bits, group_size, stream, false, pair_token,
                      pair_weight, n_tokens);
}

qmm_status qmm_moe_swiglu(const void* gate_w, const void* gate_scales, const void* gate_mins,
                          const void* up_w, const void* up_scales, const void* up_mins, const void* x,
                          const int32_t* x_rows, int64_t x_rows_count, const int32_t* expert_offsets,
                          float* h, int64_t p_rows, int64_t n_experts, int64_t n, int64_t k, int bits,
                          int group_size, void* stream) {
    return moe_common(gate_w, gate_scales, gate_mins, up_w, up_scales, up_mins, x, x_rows, x_rows_count,
                      expert_offsets, h, p_rows, n_experts, n, k, bits, group_size, stream, true);
}

static qmm_status check_batch(const qmm_gemv_desc* d, int64_t count, int bits, int group,
                              int64_t* total_rows, int64_t* kmax) {
    if (count < 0 || count > INT_LIMIT) return fail(QMM_ERR_INVALID_ARGUMENT, "count=%lld out of range", (long long)count);
    if (count > 0 && !d) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL descriptor array");
    *total_rows = 0;
    *kmax = 32;
    char why[sizeof g_err];
    for (int64_t i = 0; i < count; ++i) {
        qmm_status st = check_format(d[i].n, d[i].k, bits, group);
        if (st == QMM_OK && d[i].n > 0) st = check_weight_ptrs(d[i].w_packed, d[i].scales, d[i].mins, bits);
        if (st != QMM_OK) {
            memcpy(why, g_err, sizeof why);
            return fail(st, "descriptor %lld: %s", (long long)i, why);
        }
        if (d[i].n == 0) continue;
        if (!d[i].x || !d[i].y) return fail(QMM_ERR_INVALID_ARGUMENT, "descriptor %lld: NULL x or y", (long long)i);
        if (!aligned(d[i].x, 16) || !aligned(d[i].y, 16))
            return fail(QMM_ERR_MISALIGNED, "descriptor %lld: x or y not 16-byte aligned", (long long)i);
        *total_rows += d[i].n;
        if (d[i].k > *kmax) *kmax = d[i].k;
    }
    return QMM_OK;
}

qmm_status qmm_gemv_batch_prepare(qmm_gemv_desc* descs, int64_t count, int bits, int group_size) {
    int64_t rows = 0, kmax = 0;
    qmm_status st = check_batch(descs, count, bits, group_size, &rows, &kmax);
    if (st != QMM_OK) return st;
    GemvShape sh{};
    if (!plan_batched(rows, kmax, bits, group_size, &sh))
        return fail(QMM_ERR_UNSUPPORTED, "largest k=%lld too large for a batched launch", (long long)kmax);
    int64_t first = 0;
    for (int64_t i = 0; i < count; ++i) {
        descs[i].first_item = first;
        first += batched_items(sh, descs[i].n, descs[i].k);
    }
    return ok();
}

qmm_status qmm_gemv_batched(const qmm_gemv_desc* descs_device, const qmm_gemv_desc* descs_host,
                            int64_t count, int bits, int group_size, void* stream) {
    int64_t rows = 0, kmax = 0;
    qmm_status st = check_batch(descs_host, count, bits, group_size, &rows, &kmax);
    if (st != QMM_OK) return st;
    if (rows == 0) return ok();
    if (!descs_device || !aligned(descs_device, 8))
        return fail(QMM_ERR_INVALID_ARGUMENT, "descs_device NULL or not 8-byte aligned");
    GemvShape sh{};
    if (!plan_batched(rows, kmax, bits, group_size, &sh))
        return fail(QMM_ERR_UNSUPPORTED, "largest k=%lld too large for a batched launch", (long long)kmax);
    int64_t first = 0;
    for (int64_t i = 0; i < count; ++i) {
        if (descs_host[i].first_item != first)
            return fail(QMM_ERR_INVALID_ARGUMENT,
                        "descriptor %lld not prepared for this batch (call qmm_gemv_batch_prepare)", (long long)i);
        first += batched_items(sh, descs_host[i].n, descs_host[i].k);
    }
    if (first > INT_LIMIT) return fail(QMM_ERR_UNSUPPORTED, "more than 2^31-1 row batches in one batched launch");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    sh.work = first;
    sh.cus = cus;
    // Three 4-wave work-groups per CU, what this kernel's register count
    // lets a CU hold at once: measured on the decode projection set, 2 %
    // faster than two, and a grid sized for four (more work-groups than fit,
    // so the last ones queue) is 6 % slower.
    sh.waves_per_cu = override_or(OV_GEMV_WAVES_PER_CU, BATCHED_WAVES_PER_CU);
    BatchArgs a{reinterpret_cast<const BatchDesc*>(descs_device), (int)count, first, group_size, bits};
    a.stride = (int)((count + BATCH_COARSE - 1) / BATCH_COARSE);
    for (int j = 0; j < BATCH_COARSE; ++j) {
        const int64_t d = (int64_t)j * a.stride;
        a.coarse.first[j] = d < count ? (int)descs_host[d].first_item : INT_MAX;
    }
    return launched(launch_batched(a, sh, as_stream(stream)), "qmm_gemv_batched");
}

qmm_status qmm_unpack(const void* w_packed, uint8_t* codes, int64_t n, int64_t k, int bits,
                      void* stream) {
    qmm_status st = check_format(n, k, bits, 32);
    if (st != QMM_OK) return st;
    if (bits == 16) return fail(QMM_ERR_UNSUPPORTED, "bits=16 holds fp16 weights, not codes to unpack");
    if (n == 0) return ok();
    if (!w_packed || !codes) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL w_packed or codes");
    if (!aligned(w_packed, 16) || !aligned(codes, 16))
        return fail(QMM_ERR_MISALIGNED, "w_packed or codes not 16-byte aligned");
    int cus = 0;
    if ((st = device_cus(&cus)) != QMM_OK) return st;
    return launched(launch_unpack(static_cast<const uint32_t*>(w_packed), codes, n, k, bits,
                                  as_stream(stream)),
                    "qmm_unpack");
}

qmm_status qmm_get_plan(int op, int64_t m, int64_t n, int64_t k, int bits, int group_size,
                        int cu_count, size_t workspace_bytes, qmm_plan* plan) {
    if (!plan) return fail(QMM_ERR_INVALID_ARGUMENT, "NULL plan");
    memset(plan, 0, sizeof *plan);
    qmm_status st = check_format(n, k, bits, group_size);
    if (st != QMM_OK) return st;
    if (m < 0) return fail(QMM_ERR_INVALID_ARGUMENT, "m is negative");
    int cus = cu_count;
    if (cus <= 0 && (st = device_cus(&cus)) != QMM_OK) return st;
    plan->block = 256;
    plan->split_k = 1;
    if (op == 0 || (op == 1 && m == 1)) {
        const GemvShape sh = plan_gemv(n, k, bits, group_size, cus);
        plan->variant = 0;
        plan->lanes_per_row = sh.lpr;
        plan->units_per_lane = sh.xc;
        plan->rows_per_iter = sh.u;
        plan->unit_codes = sh.unit;
        plan->grid = sh.grid;
        plan->reserved[0] = sh.multipass;
        plan->reserved[1] = sh.staged;
        plan->reserved[2] = sh.late;
        return ok();
    }
    if (op == 3) {
        GemvShape sh{};
        if (!plan_batched(n, k, bits, group_size, &sh))
            return fail(QMM_ERR_UNSUPPORTED, "k too large for a batched launch");
        plan->variant = 3;
        plan->lanes_per_row = sh.lpr;
        plan->units_per_lane = sh.xc;
        plan->rows_per_iter = sh.u;
        plan->unit_codes = sh.unit;
        plan->grid = persistent_grid(batched_items(sh, n, k), cus, 4, BATCHED_WAVES_PER_CU);
        return ok();
    }
    if (op == 2 || (op == 1 && m <= ROWS_KERNEL_MAX_M)) {
        const RowsShape sh = plan_rows(m, n, k, bits, group_size, cus, 1);
        plan->variant = 1;
        plan->lanes_per_row = sh.lpr;
        plan->units_per_lane = sh.xc;
        plan->rows_per_iter = sh.mr;
        plan->unit_codes = sh.unit;
        plan->grid = (int64_t)sh.grid_x * sh.grid_y;
        plan->reserved[0] = sh.multipass;
        return ok();
    }
    if (op == 1) {
        const GemmShape sh = plan_gemm(m, n, k, group_size, bits, cus, workspace_bytes, nullptr);
        plan->variant = sh.kernel == 1 ? 4 : 2;
        plan->block = sh.kernel == 1 ? gemm_wl_threads(sh.tile_m) : gemm_threads(sh.tile_m);
        plan->split_k = sh.split;
        plan->tile_m = sh.tile_m;
        plan->tile_n = sh.tile_n;
        plan->grid = 8 * (((int64_t)sh.grid_m * sh.grid_n * sh.split + 7) / 8);
        return ok();
    }
    return fail(QMM_ERR_INVALID_ARGUMENT, "op=%d unknown", op);
}

}  // extern "C"
