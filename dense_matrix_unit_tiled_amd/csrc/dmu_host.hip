// C ABI of the GEMM library: argument validation, kernel selection, launch.
//
// Validation follows the host entry point of "Tensor Cores, CUTLASS and CuTe"
// section 4.4 (type, rank and layout are checked before an untyped pointer is
// reinterpreted), extended to what that entry point leaves to its caller:
// ragged sizes, any element alignment, leading dimensions and batch strides
// (section 7's strided-batched form), and aliasing of the output.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/dmu.h"
#include "dmu_host.hpp"

// ---------------------------------------------------------------------------
// Library-held scratch of dmu_gemm_streamk_noalloc: the stream-K workspace
// (error word, flags, partial-sum slots) in a file-scope device array, so that
// callers that cannot allocate (code under graph capture, tight serving loops)
// still get the schedule.  Each GPU holds its own copy, at its own address,
// until the process ends.  In host code the array's name is only a stand-in:
// its device address is asked for once per device (hipGetSymbolAddress, with
// that device current) and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[DMU_STREAMK_SCRATCH_BYTES];

namespace dmu {

static thread_local char g_err[512];

void set_error(const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = 0; }

int check_launch(const char *what)
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    return DMU_OK;
}

namespace {

struct Plan {
    bool launch;     // false: nothing to do (empty problem)
    LaunchCfg cfg;
    GemmParams p;
    int combo;       // index into the launcher table
    const char *name;
};

constexpr int64_t LIM31 = (int64_t)1 << 31;
// A problem of at most this many 128 x 128 tiles (over all batch slices) takes
// 64 x 128 tiles instead: half the compute units of the 256-unit chip this
// library is built for.  (Fixed rather than asked of the device, so that the
// choice -- and the kernel name -- is known without one.)
constexpr int64_t FEW_TILES = 128;

int elem_bytes(int t) { return (t == DMU_F32 || t == DMU_I32) ? 4 : (t == DMU_I8 || t == DMU_E4M3 ? 1 : 2); }

// Supported (in, acc, out) triples -> launcher index.
int combo_of(int in, int acc, int out)
{
    if (in == DMU_F16 && acc == DMU_F32 && out == DMU_F32) return 0;
    if (in == DMU_F16 && acc == DMU_F32 && out == DMU_F16) return 1;
    if (in == DMU_F16 && acc == DMU_F16 && out == DMU_F16) return 1; // fp32 sum, one rounding to fp16
    if (in == DMU_BF16 && acc == DMU_F32 && out == DMU_BF16) return 2;
    if (in == DMU_BF16 && acc == DMU_F32 && out == DMU_F32) return 3;
    if (in == DMU_I8 && acc == DMU_I32 && out == DMU_I32) return 4;
    if (in == DMU_I8 && acc == DMU_I32 && out == DMU_F32) return 5;  // dequantising outputs
    if (in == DMU_I8 && acc == DMU_I32 && out == DMU_F16) return 6;
    if (in == DMU_I8 && acc == DMU_I32 && out == DMU_BF16) return 7;
    if (in == DMU_E4M3 && acc == DMU_F32 && out == DMU_F32) return 8;
    if (in == DMU_E4M3 && acc == DMU_F32 && out == DMU_F16) return 9;
    if (in == DMU_E4M3 && acc == DMU_F32 && out == DMU_BF16) return 10;
    return -1;
}

constexpr int NUM_COMBOS = 11;
const char *const COMBO_NAMES[NUM_COMBOS] = {"f16_f32", "f16_f16", "bf16_bf16", "bf16_f32",
                                             "i8_i32",  "i8_f32",  "i8_f16",    "i8_bf16",
                                             "e4m3_f32", "e4m3_f16", "e4m3_bf16"};

// Names of every kernel variant, built once (thread-safe static init).
struct NameTable {
    char at[NUM_TILE_CFGS][4][4][NUM_COMBOS][48];
};

const NameTable &kernel_names()
{
    static const NameTable table = [] {
        static const char *const TILE_NAMES[] = {"256x256", "256x128", "128x128", "generic64", "256x256w4", "64x128"};
        static const char *const MODE_NAMES[] = {"k16", "kd", "t16", "t8"};
        NameTable t;
        for (int a = 0; a < NUM_TILE_CFGS; ++a)
            for (int x = 0; x < 4; ++x)
                for (int y = 0; y < 4; ++y)
                    for (int c = 0; c < NUM_COMBOS; ++c)
                        snprintf(t.at[a][x][y][c], sizeof(t.at[a][x][y][c]), "mfma_%s_%s_%s_%s", TILE_NAMES[a],
                                 a == TILE_GENERIC ? "any" : MODE_NAMES[x], a == TILE_GENERIC ? "any" : MODE_NAMES[y],
                                 COMBO_NAMES[c]);
        return t;
    }();
    return table;
}

// Elements spanned by a rows x cols matrix stored with `layout` and `ld`.
int64_t extent(int layout, int64_t rows, int64_t cols, int64_t ld)
{
    if (rows == 0 || cols == 0)
        return 0;
    return layout == DMU_ROW_MAJOR ? (rows - 1) * ld + cols : (cols - 1) * ld + rows;
}

// Byte range [lo, hi) covered by all batch slices of an operand.
void span(const void *ptr, int64_t stride, int64_t batch, int64_t ext, int esz, uintptr_t *lo, uintptr_t *hi)
{
    *lo = (uintptr_t)ptr;
    *hi = *lo + (uintptr_t)(((batch - 1) * stride + ext) * esz);
}

bool overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) { return a0 < b1 && b0 < a1; }

bool aligned(const void *p, int64_t ld, int64_t stride, int esz, int vb)
{
    return ((uintptr_t)p % vb) == 0 && (ld * esz) % vb == 0 && (stride * esz) % vb == 0;
}

// Load mode of one operand: -1 if only the generic kernel can read it.
//  kc: K is the contiguous dimension; mn: the operand's M (or N) size.
int operand_mode(bool kc, const void *p, int64_t ld, int64_t stride, int esz, int64_t K, int64_t mn)
{
    if (kc) {
        if (aligned(p, ld, stride, esz, 16) && (K * esz) % 16 == 0)
            return KC16;
        if (aligned(p, ld, stride, esz, 4))
            return KCD;
        return -1;
    }
    if (esz == 2 && aligned(p, ld, stride, esz, 16) && mn % 8 == 0)
        return MC16;
    if (esz == 1 && aligned(p, ld, stride, esz, 16) && mn % 16 == 0)
        return MC8;
    return -1;
}

int validate_epilogue(const dmu_gemm_args *a, const dmu_epilogue *ep, Plan *plan);

int validate(const dmu_gemm_args *a, Plan *plan)
{
    memset(plan, 0, sizeof(*plan));
    if (!a) {
        set_error("args is NULL");
        return DMU_ERR_INVALID_ARG;
    }
    if (a->M < 0 || a->N < 0 || a->K < 0 || a->batch < 0) {
        set_error("negative size (M=%lld N=%lld K=%lld batch=%lld)", (long long)a->M, (long long)a->N,
                  (long long)a->K, (long long)a->batch);
        return DMU_ERR_INVALID_ARG;
    }
    if (a->M >= LIM31 || a->N >= LIM31 || a->K >= LIM31 || a->batch >= LIM31) {
        set_error("size of 2^31 or more is not supported");
        return DMU_ERR_UNSUPPORTED;
    }
    const int combo = combo_of(a->in_type, a->acc_type, a->out_type);
    if (combo < 0) {
        set_error("unsupported (in, acc, out) types (%d, %d, %d)", a->in_type, a->acc_type, a->out_type);
        return DMU_ERR_UNSUPPORTED;
    }
    if ((a->layout_a != DMU_ROW_MAJOR && a->layout_a != DMU_COL_MAJOR) ||
        (a->layout_b != DMU_ROW_MAJOR && a->layout_b != DMU_COL_MAJOR)) {
        set_error("layout must be DMU_ROW_MAJOR or DMU_COL_MAJOR");
        return DMU_ERR_INVALID_ARG;
    }
    if (a->stride_a < 0 || a->stride_b < 0 || a->stride_c < 0 || a->stride_d < 0) {
        set_error("negative batch stride");
        return DMU_ERR_INVALID_ARG;
    }
    plan->combo = combo;
    if (a->M == 0 || a->N == 0 || a->batch == 0) {
        plan->launch = false;
        return DMU_OK;
    }
    const int64_t M = a->M, N = a->N, K = a->K, batch = a->batch;
    const int esz = elem_bytes(a->in_type), osz = elem_bytes(a->out_type);
    // leading dimensions (BLAS rule: at least the contiguous extent, at least 1)
    const int64_t need_lda = a->layout_a == DMU_ROW_MAJOR ? K : M;
    const int64_t need_ldb = a->layout_b == DMU_ROW_MAJOR ? N : K;
    if (a->lda < (need_lda > 1 ? need_lda : 1) || a->ldb < (need_ldb > 1 ? need_ldb : 1)) {
        set_error("lda=%lld / ldb=%lld below the contiguous extent (%lld / %lld)", (long long)a->lda,
                  (long long)a->ldb, (long long)need_lda, (long long)need_ldb);
        return DMU_ERR_INVALID_ARG;
    }
    if (a->ldd < N || (a->C && a->ldc < N)) {
        set_error("ldd=%lld / ldc=%lld below N=%lld", (long long)a->ldd, (long long)a->ldc, (long long)N);
        return DMU_ERR_INVALID_ARG;
    }
    if (!a->D || (K > 0 && (!a->A || !a->B))) {
        set_error("NULL operand pointer");
        return DMU_ERR_INVALID_ARG;
    }
    const int64_t ext_d = extent(DMU_ROW_MAJOR, M, N, a->ldd);
    if (batch > 1 && a->stride_d < ext_d) {
        set_error("stride_d=%lld lets batch slices of D overlap (needs >= %lld)", (long long)a->stride_d,
                  (long long)ext_d);
        return DMU_ERR_INVALID_ARG;
    }
    // aliasing: D must not overlap A or B; C may only coincide with D exactly
    uintptr_t d0, d1;
    span(a->D, a->stride_d, batch, ext_d, osz, &d0, &d1);
    if (K > 0) {
        uintptr_t x0, x1;
        span(a->A, a->stride_a, batch, extent(a->layout_a, M, K, a->lda), esz, &x0, &x1);
        if (overlap(d0, d1, x0, x1)) {
            set_error("D overlaps A");
            return DMU_ERR_INVALID_ARG;
        }
        span(a->B, a->stride_b, batch, extent(a->layout_b, K, N, a->ldb), esz, &x0, &x1);
        if (overlap(d0, d1, x0, x1)) {
            set_error("D overlaps B");
            return DMU_ERR_INVALID_ARG;
        }
    }
    if (a->C) {
        uintptr_t c0, c1;
        span(a->C, a->stride_c, batch, extent(DMU_ROW_MAJOR, M, N, a->ldc), osz, &c0, &c1);
        const bool same = a->C == a->D && a->ldc == a->ldd && a->stride_c == a->stride_d;
        if (!same && overlap(d0, d1, c0, c1)) {
            set_error("C partially overlaps D (only C == D with equal ldc/stride is allowed)");
            return DMU_ERR_INVALID_ARG;
        }
    }
    if (((uintptr_t)a->D % osz) || (a->C && ((uintptr_t)a->C % osz)) || ((uintptr_t)a->A % esz) ||
        ((uintptr_t)a->B % esz)) {
        set_error("pointer not aligned to its element size");
        return DMU_ERR_INVALID_ARG;
    }

    // kernel selection
    const bool a_kc = a->layout_a == DMU_ROW_MAJOR, b_kc = a->layout_b == DMU_COL_MAJOR;
    int amode = K > 0 ? operand_mode(a_kc, a->A, a->lda, batch > 1 ? a->stride_a : 0, esz, K, M) : -1;
    int bmode = K > 0 ? operand_mode(b_kc, a->B, a->ldb, batch > 1 ? a->stride_b : 0, esz, K, N) : -1;
    if (amode >= 0 && extent(a->layout_a, M, K, a->lda) * esz >= ((int64_t)1 << 31))
        amode = -1; // slice too large for one buffer descriptor
    if (bmode >= 0 && extent(a->layout_b, K, N, a->ldb) * esz >= ((int64_t)1 << 31))
        bmode = -1;
    int tile = TILE_GENERIC;
    const char *env = getenv("DMU_FORCE_KERNEL");
    const bool force_generic = env && strcmp(env, "generic") == 0;
    if (amode >= 0 && bmode >= 0 && !force_generic) {
        const int64_t big = ((M + 255) / 256) * ((N + 255) / 256) * batch;
        const int64_t nk = (K * esz + 127) / 128; // K-tiles
        if (N <= 128 && M > 128)
            tile = TILE_256x128;
        else if (big >= 240)
            // Two K-tiles or fewer: each tile is little more than its
            // epilogue, and the 256 x 128 tile (two K-tiles in flight, half
            // the D per tile) is faster (batch 32 x 4096 x 4096 x 128 fp16 ->
            // fp32: 427 -> 401 us); from four K-tiles on, 256 x 256 is
            // faster or equal (same shape with K = 256: 482 vs 531 us).
            tile = nk <= 2 ? TILE_256x128 : TILE_256x256;
        else
            tile = TILE_128x128;
        // Few tiles: 64 x 128 tiles put twice as many workgroups on the compute
        // units (up to all 256 of the chip) at a somewhat lower rate per unit
        // (1024 x 1024 x 16384 bf16, 64 tiles of 128 x 128: 114.0 -> 81.2 us, same
        // bits).  The 64-row tile takes K-contiguous A only.
        const bool a_kc_mode = amode == KC16 || amode == KCD;
        if (tile == TILE_128x128 && a_kc_mode && ((M + 127) / 128) * ((N + 127) / 128) * batch <= FEW_TILES)
            tile = TILE_64x128;
        // (The four-wavefront 256 x 256 tile, a third fewer LDS fragment bytes
        // per flop, is not chosen by default: measured in interleaved pairs on
        // one box, 4096^3 bf16 NN 99.0 us on eight wavefronts against 99.6 us,
        // 8192^3 int8 TN 424 against 434 us, 5000 x 3000 x 2050 fp16 TN 66
        // against 72 us.  DMU_FORCE_KERNEL=256x256w4 selects it.)
        if (env && strcmp(env, "256x256") == 0) tile = TILE_256x256;
        if (env && strcmp(env, "256x256w4") == 0) tile = TILE_256x256W4;
        if (env && strcmp(env, "256x128") == 0) tile = TILE_256x128;
        if (env && strcmp(env, "128x128") == 0) tile = TILE_128x128;
        if (env && strcmp(env, "64x128") == 0 && a_kc_mode) tile = TILE_64x128;
        if (a->in_type == DMU_E4M3 && (tile == TILE_256x256 || tile == TILE_256x256W4))
            tile = TILE_256x128; // e4m3 fragments need the registers of a 64 x 64 wavefront tile
        if (a->in_type == DMU_I8 && tile == TILE_256x256W4)
            tile = TILE_256x256; // the four-wavefront tile is built for 16-bit inputs only
    }
    const int64_t bm = tile_bm(tile), bn = tile_bn(tile);
    const int64_t tm = (M + bm - 1) / bm, tn = (N + bn - 1) / bn;
    if (tm * tn * batch >= ((int64_t)1 << 32)) {
        set_error("too many tiles for one launch");
        return DMU_ERR_UNSUPPORTED;
    }
    plan->launch = true;
    plan->cfg.tile = tile;
    plan->cfg.amode = amode < 0 ? 0 : amode;
    plan->cfg.bmode = bmode < 0 ? 0 : bmode;
    plan->cfg.workers = 0;
    plan->name = kernel_names().at[tile][plan->cfg.amode][plan->cfg.bmode][combo];
    GemmParams &p = plan->p;
    p.A = static_cast<const char *>(a->A);
    p.B = static_cast<const char *>(a->B);
    p.C = static_cast<const char *>(a->C);
    p.D = static_cast<char *>(a->D);
    p.lda = a->lda;
    p.ldb = a->ldb;
    p.ldc = a->ldc;
    p.ldd = a->ldd;
    p.stride_a = batch > 1 ? a->stride_a : 0;
    p.stride_b = batch > 1 ? a->stride_b : 0;
    p.stride_c = batch > 1 ? a->stride_c : 0;
    p.stride_d = batch > 1 ? a->stride_d : 0;
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.batch = (int32_t)batch;
    p.tiles_m = (int32_t)tm;
    p.tiles_n = (int32_t)tn;
    p.total_tiles = (uint32_t)(tm * tn * batch);
    p.a_kc = a_kc;
    p.b_kc = b_kc;
    const bool c_vec = !a->C || (((uintptr_t)a->C % (4 * osz)) == 0 && a->ldc % 4 == 0 && p.stride_c % 4 == 0);
    p.d_vec4 = ((uintptr_t)a->D % (4 * osz)) == 0 && a->ldd % 4 == 0 && p.stride_d % 4 == 0 && c_vec;
    p.d_nt = ((uintptr_t)a->D % 128) == 0 && (a->ldd * osz) % 128 == 0 && (p.stride_d * osz) % 128 == 0;
    p.a_bytes = extent(a->layout_a, M, K, a->lda) * esz;
    p.b_bytes = extent(a->layout_b, K, N, a->ldb) * esz;
    return DMU_OK;
}

// The fused epilogue's operands, checked after the product's (plan filled by validate).
int validate_epilogue(const dmu_gemm_args *a, const dmu_epilogue *ep, Plan *plan)
{
    if (!ep)
        return DMU_OK;
    if (ep->act < DMU_ACT_NONE || ep->act > DMU_ACT_GELU_TANH) {
        set_error("epilogue activation %d is not DMU_ACT_NONE, DMU_ACT_RELU or DMU_ACT_GELU_TANH", ep->act);
        return DMU_ERR_INVALID_ARG;
    }
    const bool any = ep->row_scale || ep->col_scale || ep->bias || ep->act != DMU_ACT_NONE;
    if (any && a->out_type == DMU_I32) {
        set_error("int32 output takes no epilogue");
        return DMU_ERR_UNSUPPORTED;
    }
    if (ep->stride_row_scale < 0 || ep->stride_col_scale < 0 || ep->stride_bias < 0) {
        set_error("negative epilogue vector stride");
        return DMU_ERR_INVALID_ARG;
    }
    if (((uintptr_t)ep->row_scale % 4) || ((uintptr_t)ep->col_scale % 4) || ((uintptr_t)ep->bias % 4)) {
        set_error("epilogue vector not aligned to 4 bytes");
        return DMU_ERR_INVALID_ARG;
    }
    if (plan->launch) { // vectors are inputs: they may not overlap the output
        const int64_t batch = a->batch;
        uintptr_t d0, d1;
        span(a->D, batch > 1 ? a->stride_d : 0, batch, extent(DMU_ROW_MAJOR, a->M, a->N, a->ldd),
             elem_bytes(a->out_type), &d0, &d1);
        const struct { const float *v; int64_t stride, n; const char *what; } vecs[3] = {
            {ep->row_scale, ep->stride_row_scale, a->M, "row_scale"},
            {ep->col_scale, ep->stride_col_scale, a->N, "col_scale"},
            {ep->bias, ep->stride_bias, a->N, "bias"}};
        for (const auto &v : vecs) {
            if (!v.v)
                continue;
            uintptr_t x0, x1;
            span(v.v, batch > 1 ? v.stride : 0, batch, v.n, 4, &x0, &x1);
            if (overlap(d0, d1, x0, x1)) {
                set_error("epilogue %s overlaps D", v.what);
                return DMU_ERR_INVALID_ARG;
            }
        }
    }
    GemmParams &p = plan->p;
    p.rs = ep->row_scale;
    p.cs = ep->col_scale;
    p.bias = ep->bias;
    p.stride_rs = a->batch > 1 ? ep->stride_row_scale : 0;
    p.stride_cs = a->batch > 1 ? ep->stride_col_scale : 0;
    p.stride_bias = a->batch > 1 ? ep->stride_bias : 0;
    p.act = ep->act;
    p.epi = (ep->row_scale || ep->col_scale || ep->bias) ? 1 : 0;
    return DMU_OK;
}

// Stream-K workspace layout: the error word (first 256 bytes), the flags (one
// 32-bit word per worker, from byte 256), then one BM x BN slot of 32-bit
// accumulators per worker (from the next multiple of 256 bytes).
struct SkLayout {
    uint32_t workers; // 0: the call runs the data-parallel kernel
    uint32_t nk, q, r; // K-tiles per tile; iterations = q workers + r
    size_t flags_off, partials_off, slot_bytes, bytes;
};

constexpr uint32_t SK_SPIN_LIMIT = 1u << 22; // polls (each after a short sleep), well over a second

// Polls of a flag before a wait gives up: SK_SPIN_LIMIT, or DMU_STREAMK_SPIN_LIMIT
// (a test hook: a tiny limit makes the waits give up while every kernel still
// exits normally).
uint32_t sk_spin_limit()
{
    const char *env = getenv("DMU_STREAMK_SPIN_LIMIT");
    if (!env || !*env)
        return SK_SPIN_LIMIT;
    char *end = nullptr;
    const unsigned long v = strtoul(env, &end, 10);
    return (end && *end == 0 && v <= SK_SPIN_LIMIT) ? (uint32_t)v : SK_SPIN_LIMIT;
}

// Stream-K runs the 256 x 128 tile where the data-parallel plan has 256 x 256,
// and the 128 x 128 tile where it has 64 x 128.
void sk_retile(Plan *plan, const dmu_gemm_args *a)
{
    if (!plan->launch)
        return;
    int to;
    if (plan->cfg.tile == TILE_256x256 || plan->cfg.tile == TILE_256x256W4)
        to = TILE_256x128;
    else if (plan->cfg.tile == TILE_64x128)
        to = TILE_128x128;
    else
        return;
    const int64_t tm = (a->M + tile_bm(to) - 1) / tile_bm(to), tn = (a->N + tile_bn(to) - 1) / tile_bn(to);
    if (tm * tn * a->batch >= ((int64_t)1 << 31))
        return; // too many iterations for the 32-bit schedule anyway: stays data-parallel
    plan->cfg.tile = to;
    plan->p.tiles_m = (int32_t)tm;
    plan->p.tiles_n = (int32_t)tn;
    plan->p.total_tiles = (uint32_t)(tm * tn * a->batch);
    plan->name = kernel_names().at[plan->cfg.tile][plan->cfg.amode][plan->cfg.bmode][plan->combo];
}

// Compute units of the current device, asked once per device.
int device_cus(const char *who, int *out)
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        set_error("%s: no current HIP device", who);
        return DMU_ERR_HIP;
    }
    if (__atomic_load_n(&cus[dev], __ATOMIC_RELAXED) == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            set_error("%s: cannot read the compute-unit count", who);
            return DMU_ERR_HIP;
        }
        __atomic_store_n(&cus[dev], n, __ATOMIC_RELAXED);
    }
    *out = __atomic_load_n(&cus[dev], __ATOMIC_RELAXED);
    return DMU_OK;
}

// The persistent form of the tiled kernel (gemm_persist: one workgroup per
// compute unit loops over the tiles and loads the next tile's first K-tile
// before the current tile's epilogue) replaces the one-workgroup-per-tile
// launch for short K loops (at most four K-tiles) with at least four tiles per
// compute unit, where the per-tile start-up and the launch of each workgroup
// weigh most (measured on the 256-unit chip, same box: batch 32 x 4096 x 4096
// x 128 fp16 -> fp32, 64 tiles of two K-tiles per unit, 405.8 -> 379.6 us;
// long loops lose a little: 8192^3 int8, 4 tiles of 64 K-tiles per unit,
// 425.7 -> 428.2 us; 8192^3 e4m3, 8 per unit, 435.9 -> 440.4 us).
// With K of at most two K-tiles (the whole range loaded before the previous
// tile's epilogue) two tiles per unit already pay: 4096 x 4096 x 128 fp16 ->
// fp32, 512 tiles, 19.1 -> 18.5 us; 4096 x 4096 x 64, 17.0 -> 16.3 us.
// DMU_PERSIST=always or never overrides the choice (tests and sweeps).
constexpr int64_t PERSIST_MIN_TILES_PER_CU = 4, PERSIST_MIN_TILES_PER_CU_SHORT = 2, PERSIST_MAX_KTILES = 4;

int persist_layout(Plan *plan, const dmu_gemm_args *a)
{
    plan->cfg.workers = 0;
    if (!plan->launch || plan->cfg.tile == TILE_GENERIC || plan->cfg.tile == TILE_256x256W4 ||
        plan->cfg.tile == TILE_64x128 || a->K == 0)
        return DMU_OK; // (the four-wavefront and 64-row tiles have no persistent form)
    const char *mode = getenv("DMU_PERSIST");
    if (mode && strcmp(mode, "never") == 0)
        return DMU_OK;
    int cus = 0;
    const int rc = device_cus("dmu_gemm", &cus);
    if (rc != DMU_OK)
        return rc;
    const int64_t tiles = plan->p.total_tiles, nk = (a->K * elem_bytes(a->in_type) + 127) / 128;
    const bool always = mode && strcmp(mode, "always") == 0;
    // (the short-K form exists for the tiles with two staging sets, not for e4m3)
    const bool short_form = nk <= 2 && a->in_type != DMU_E4M3 &&
                            (plan->cfg.tile == TILE_256x128 || plan->cfg.tile == TILE_128x128);
    const int64_t min_per_cu = short_form ? PERSIST_MIN_TILES_PER_CU_SHORT : PERSIST_MIN_TILES_PER_CU;
    if (!always && (tiles < min_per_cu * cus || nk > PERSIST_MAX_KTILES))
        return DMU_OK;
    // one workgroup per compute unit, a multiple of the 8 XCDs so that each
    // worker's tiles stay on its XCD; never more workers than tiles
    int64_t w = cus >= 8 ? (cus / 8) * 8 : cus;
    if (w > tiles)
        w = tiles;
    plan->cfg.workers = (int)w;
    return DMU_OK;
}

// Stream-K pays when the data-parallel tiles leave compute units idle: it is
// chosen when those tiles fill less than 80 % of their waves (measured on the
// 256-unit chip: 1024 x 1024 x 16384 bf16, 64 tiles, 123 -> 50 us; the
// 5000 x 3000 x 2050 problem, 240 tiles = 94 %, stays data-parallel: stream-K
// on its 480 smaller tiles took 97 us against 73 us).  Where the data-parallel
// plan has 64 x 128 tiles, those already spread a few-tile problem over more
// units, and stream-K (on 128 x 128) pays only below 60 % (bf16, interleaved:
// 1024 x 1024 x 4096, 128 tiles = 50 %, 24.4 -> 21.0 us; 1280 x 1024 x 8192,
// 160 = 63 %, 43.7 against 48.2 us; 1280^2 x 8192, 200 = 78 %, 47.3 against
// 51.7 us).  DMU_STREAMK=always or never overrides the choice (tests and
// sweeps).
constexpr double SK_MIN_IDLE_FILL = 0.8, SK_MIN_IDLE_FILL_64 = 0.6;

int sk_layout(Plan *plan, const dmu_gemm_args *a, SkLayout *sk)
{
    memset(sk, 0, sizeof(*sk));
    if (!plan->launch || plan->cfg.tile == TILE_GENERIC)
        return DMU_OK;
    const char *mode = getenv("DMU_STREAMK");
    if (mode && strcmp(mode, "never") == 0)
        return DMU_OK;
    const int64_t nk = (a->K * elem_bytes(a->in_type) + 127) / 128;
    if (nk == 0)
        return DMU_OK; // K == 0: D = C, data-parallel
    int cu_count = 0;
    const int crc = device_cus("dmu_gemm_streamk", &cu_count);
    if (crc != DMU_OK)
        return crc;
    const uint64_t n = (uint64_t)cu_count;
    if (!(mode && strcmp(mode, "always") == 0)) {
        const uint64_t tiles = plan->p.total_tiles, waves = (tiles + n - 1) / n;
        const double min_fill = plan->cfg.tile == TILE_64x128 ? SK_MIN_IDLE_FILL_64 : SK_MIN_IDLE_FILL;
        if ((double)tiles >= min_fill * (double)(waves * n))
            return DMU_OK; // the data-parallel waves are full enough
    }
    sk_retile(plan, a);
    const Plan &pl = *plan;
    if (pl.cfg.tile == TILE_256x256 || pl.cfg.tile == TILE_256x256W4 || pl.cfg.tile == TILE_64x128)
        return DMU_OK; // too many tiles to retile: data-parallel
    const uint64_t iters = (uint64_t)pl.p.total_tiles * (uint64_t)nk;
    if (iters >= ((uint64_t)1 << 31))
        return DMU_OK; // more iterations than the 32-bit schedule counts: data-parallel
    sk->workers = (uint32_t)(iters < n ? iters : n);
    sk->nk = (uint32_t)nk;
    sk->q = (uint32_t)(iters / sk->workers);
    sk->r = (uint32_t)(iters % sk->workers);
    sk->slot_bytes = (size_t)tile_bm(pl.cfg.tile) * tile_bn(pl.cfg.tile) * 4;
    sk->flags_off = 256;
    sk->partials_off = (sk->flags_off + (size_t)sk->workers * 4 + 255) & ~(size_t)255;
    sk->bytes = sk->partials_off + (size_t)sk->workers * sk->slot_bytes;
    return DMU_OK;
}

// The stream-K kernel's view of a workspace laid out as `sk` describes.
StreamKParams sk_params(const SkLayout &sk, char *w)
{
    StreamKParams k;
    k.error = reinterpret_cast<uint32_t *>(w);
    k.flags = reinterpret_cast<uint32_t *>(w + sk.flags_off);
    k.partials = w + sk.partials_off;
    k.workers = sk.workers;
    k.nk = sk.nk;
    k.q = sk.q;
    k.r = sk.r;
    k.spin_limit = sk_spin_limit();
    return k;
}

hipError_t launch_plan(const Plan &plan, hipStream_t s)
{
    switch (plan.combo) {
    case 0: return launch_f16_f32(plan.cfg, plan.p, s);
    case 1: return launch_f16_f16(plan.cfg, plan.p, s);
    case 2: return launch_bf16_bf16(plan.cfg, plan.p, s);
    case 3: return launch_bf16_f32(plan.cfg, plan.p, s);
    case 4: return launch_i8_i32(plan.cfg, plan.p, s);
    case 5: return launch_i8_f32(plan.cfg, plan.p, s);
    case 6: return launch_i8_f16(plan.cfg, plan.p, s);
    case 7: return launch_i8_bf16(plan.cfg, plan.p, s);
    case 8: return launch_e4m3_f32(plan.cfg, plan.p, s);
    case 9: return launch_e4m3_f16(plan.cfg, plan.p, s);
    default: return launch_e4m3_bf16(plan.cfg, plan.p, s);
    }
}

hipError_t launch_plan_sk(const Plan &plan, const StreamKParams &k, hipStream_t s)
{
    switch (plan.combo) {
    case 0: return launch_f16_f32_sk(plan.cfg, plan.p, k, s);
    case 1: return launch_f16_f16_sk(plan.cfg, plan.p, k, s);
    case 2: return launch_bf16_bf16_sk(plan.cfg, plan.p, k, s);
    case 3: return launch_bf16_f32_sk(plan.cfg, plan.p, k, s);
    case 4: return launch_i8_i32_sk(plan.cfg, plan.p, k, s);
    case 5: return launch_i8_f32_sk(plan.cfg, plan.p, k, s);
    case 6: return launch_i8_f16_sk(plan.cfg, plan.p, k, s);
    case 7: return launch_i8_bf16_sk(plan.cfg, plan.p, k, s);
    case 8: return launch_e4m3_f32_sk(plan.cfg, plan.p, k, s);
    case 9: return launch_e4m3_f16_sk(plan.cfg, plan.p, k, s);
    default: return launch_e4m3_bf16_sk(plan.cfg, plan.p, k, s);
    }
}

// The workspace may not overlap any operand.
bool workspace_overlaps(const dmu_gemm_args *a, const void *ws, size_t bytes)
{
    const uintptr_t w0 = (uintptr_t)ws, w1 = w0 + bytes;
    const int64_t batch = a->batch, esz = elem_bytes(a->in_type), osz = elem_bytes(a->out_type);
    uintptr_t x0, x1;
    span(a->D, batch > 1 ? a->stride_d : 0, batch, extent(DMU_ROW_MAJOR, a->M, a->N, a->ldd), (int)osz, &x0, &x1);
    if (overlap(w0, w1, x0, x1))
        return true;
    if (a->C) {
        span(a->C, batch > 1 ? a->stride_c : 0, batch, extent(DMU_ROW_MAJOR, a->M, a->N, a->ldc), (int)osz, &x0, &x1);
        if (overlap(w0, w1, x0, x1))
            return true;
    }
    if (a->K > 0) {
        span(a->A, batch > 1 ? a->stride_a : 0, batch, extent(a->layout_a, a->M, a->K, a->lda), (int)esz, &x0, &x1);
        if (overlap(w0, w1, x0, x1))
            return true;
        span(a->B, batch > 1 ? a->stride_b : 0, batch, extent(a->layout_b, a->K, a->N, a->ldb), (int)esz, &x0, &x1);
        if (overlap(w0, w1, x0, x1))
            return true;
    }
    return false;
}

// Device address of the library scratch (the file-scope array above) on each device.
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char *g_scratch[MAX_DEVICES]; // device address of `scratch` per device (nullptr: not asked yet)

int scratch_of_current_device(const char *who, char **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        set_error("%s: no current HIP device", who);
        return DMU_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            set_error("%s: address of the library scratch: %s", who, hipGetErrorString(e));
            return DMU_ERR_HIP;
        }
        g_scratch[dev] = static_cast<char *>(p);
    }
    *out = g_scratch[dev];
    return DMU_OK;
}

// Phase log (diagnostics): the caller's device buffer, written by every GEMM
// launch of the process while set (dmu_phase_log).
std::mutex g_phase_mu;
uint64_t *g_phase_log = nullptr;
size_t g_phase_cap = 0;  // records the buffer holds
size_t g_phase_last = 0; // records the last launch wrote
int g_phase_kind = 0;    // how they are indexed (dmu_phase_log_last)

// Points the launch at the phase log if one is set: one record per workgroup of
// the one-per-tile kernel, per tile of the persistent kernel or per stream-K
// worker (`sk_workers` > 0); none for the fallback.
int phase_attach(Plan *plan, uint32_t sk_workers, const char *who)
{
    size_t n = 0;
    int kind = 0;
    if (sk_workers > 0) {
        n = sk_workers;
        kind = 3;
    } else if (plan->cfg.tile != TILE_GENERIC) {
        n = plan->p.total_tiles;
        kind = plan->cfg.workers > 0 ? 2 : 1;
    }
    return phase_reserve(n, kind, who, &plan->p.phases);
}

// Zeroes n 32-bit words (a kernel rather than hipMemsetAsync, so that the call
// can be captured into a graph).
__global__ void __launch_bounds__(256) zero_words(uint32_t *w, uint32_t n)
{
    for (uint32_t i = threadIdx.x; i < n; i += 256)
        w[i] = 0;
}

} // namespace

int phase_reserve(size_t records, int kind, const char *who, uint64_t **log)
{
    std::lock_guard<std::mutex> lock(g_phase_mu);
    *log = nullptr;
    if (!g_phase_log)
        return DMU_OK;
    if (records > g_phase_cap) {
        set_error("%s: the launch writes %zu phase records, the log holds %zu", who, records, g_phase_cap);
        return DMU_ERR_INVALID_ARG;
    }
    if (records > 0)
        *log = g_phase_log;
    g_phase_last = records;
    g_phase_kind = kind;
    return DMU_OK;
}

} // namespace dmu

using namespace dmu;

extern "C" int dmu_gemm_check(const dmu_gemm_args *args)
{
    clear_error();
    Plan plan;
    return validate(args, &plan);
}

extern "C" const char *dmu_gemm_kernel_name(const dmu_gemm_args *args)
{
    clear_error();
    Plan plan;
    if (validate(args, &plan) != DMU_OK || !plan.launch)
        return nullptr;
    return plan.name;
}

extern "C" int dmu_gemm_ex_check(const dmu_gemm_args *args, const dmu_epilogue *ep)
{
    clear_error();
    Plan plan;
    int rc = validate(args, &plan);
    if (rc == DMU_OK)
        rc = validate_epilogue(args, ep, &plan);
    return rc;
}

extern "C" int dmu_gemm_ex(const dmu_gemm_args *args, const dmu_epilogue *ep, void *stream)
{
    clear_error();
    Plan plan;
    int rc = validate(args, &plan);
    if (rc == DMU_OK)
        rc = validate_epilogue(args, ep, &plan);
    if (rc != DMU_OK || !plan.launch)
        return rc;
    if ((rc = persist_layout(&plan, args)) != DMU_OK)
        return rc;
    if ((rc = phase_attach(&plan, 0, "dmu_gemm")) != DMU_OK)
        return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const hipError_t e = launch_plan(plan, s);
    if (e != hipSuccess) {
        set_error("dmu_gemm: launch of %s failed: %s", plan.name, hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    return DMU_OK;
}

extern "C" int dmu_gemm(const dmu_gemm_args *args, void *stream) { return dmu_gemm_ex(args, nullptr, stream); }

extern "C" int dmu_gemm_streamk_workspace_size(const dmu_gemm_args *args, size_t *bytes)
{
    clear_error();
    if (!bytes) {
        set_error("bytes is NULL");
        return DMU_ERR_INVALID_ARG;
    }
    *bytes = 0;
    Plan plan;
    int rc = validate(args, &plan);
    if (rc != DMU_OK)
        return rc;
    SkLayout sk;
    rc = sk_layout(&plan, args, &sk);
    if (rc == DMU_OK)
        *bytes = sk.bytes;
    return rc;
}

extern "C" int dmu_gemm_streamk(const dmu_gemm_args *args, const dmu_epilogue *ep, void *workspace,
                                size_t workspace_bytes, void *stream)
{
    clear_error();
    Plan plan;
    int rc = validate(args, &plan);
    if (rc == DMU_OK)
        rc = validate_epilogue(args, ep, &plan);
    if (rc != DMU_OK || !plan.launch)
        return rc;
    SkLayout sk;
    if ((rc = sk_layout(&plan, args, &sk)) != DMU_OK)
        return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (sk.workers == 0) { // the fallback kernel, or K == 0: the data-parallel launch
        if ((rc = persist_layout(&plan, args)) != DMU_OK)
            return rc;
        if ((rc = phase_attach(&plan, 0, "dmu_gemm_streamk")) != DMU_OK)
            return rc;
        e = launch_plan(plan, s);
    } else {
        if (!workspace || ((uintptr_t)workspace % 256) || workspace_bytes < sk.bytes) {
            set_error("dmu_gemm_streamk: workspace must be 256-byte aligned and hold %zu bytes", sk.bytes);
            return DMU_ERR_INVALID_ARG;
        }
        if (workspace_overlaps(args, workspace, sk.bytes)) {
            set_error("dmu_gemm_streamk: the workspace overlaps an operand");
            return DMU_ERR_INVALID_ARG;
        }
        if ((rc = phase_attach(&plan, sk.workers, "dmu_gemm_streamk")) != DMU_OK)
            return rc;
        e = launch_plan_sk(plan, sk_params(sk, static_cast<char *>(workspace)), s);
    }
    if (e != hipSuccess) {
        set_error("dmu_gemm_streamk: launch of %s failed: %s", plan.name, hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    return DMU_OK;
}

extern "C" int dmu_gemm_streamk_noalloc(const dmu_gemm_args *args, const dmu_epilogue *ep, void *stream)
{
    clear_error();
    Plan plan;
    int rc = validate(args, &plan);
    if (rc == DMU_OK)
        rc = validate_epilogue(args, ep, &plan);
    if (rc != DMU_OK || !plan.launch)
        return rc;
    SkLayout sk;
    if ((rc = sk_layout(&plan, args, &sk)) != DMU_OK)
        return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    if (sk.workers == 0) { // the data-parallel kernel: no scratch
        if ((rc = persist_layout(&plan, args)) != DMU_OK)
            return rc;
        if ((rc = phase_attach(&plan, 0, "dmu_gemm_streamk_noalloc")) != DMU_OK)
            return rc;
        e = launch_plan(plan, s);
    } else {
        if (sk.bytes > (size_t)DMU_STREAMK_SCRATCH_BYTES) {
            set_error("dmu_gemm_streamk_noalloc: the schedule needs %zu bytes of scratch, more than the "
                      "library's %zu (use dmu_gemm_streamk with a workspace)",
                      sk.bytes, (size_t)DMU_STREAMK_SCRATCH_BYTES);
            return DMU_ERR_UNSUPPORTED;
        }
        if ((rc = phase_attach(&plan, sk.workers, "dmu_gemm_streamk_noalloc")) != DMU_OK)
            return rc;
        char *w = nullptr;
        if ((rc = scratch_of_current_device("dmu_gemm_streamk_noalloc", &w)) != DMU_OK)
            return rc;
        // the error word and the flags start at zero: a failed earlier call may have left them set
        const uint32_t nwords = (uint32_t)(sk.partials_off / 4);
        hipLaunchKernelGGL(zero_words, dim3(1), dim3(256), 0, s, reinterpret_cast<uint32_t *>(w), nwords);
        e = hipGetLastError();
        if (e == hipSuccess)
            e = launch_plan_sk(plan, sk_params(sk, w), s);
    }
    if (e != hipSuccess) {
        set_error("dmu_gemm_streamk_noalloc: launch of %s failed: %s", plan.name, hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    return DMU_OK;
}

extern "C" int dmu_gemm_streamk_error(const void *workspace, void *stream, int *failed)
{
    clear_error();
    if (!failed) {
        set_error("dmu_gemm_streamk_error: NULL failed");
        return DMU_ERR_INVALID_ARG;
    }
    *failed = 0;
    if ((uintptr_t)workspace % 256) {
        set_error("dmu_gemm_streamk_error: workspace is not 256-byte aligned");
        return DMU_ERR_INVALID_ARG;
    }
    if (!workspace) { // the library scratch of dmu_gemm_streamk_noalloc on the current device
        char *w = nullptr;
        const int rc = scratch_of_current_device("dmu_gemm_streamk_error", &w);
        if (rc != DMU_OK)
            return rc;
        workspace = w;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        set_error("dmu_gemm_streamk_error: %s", hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    *failed = word != 0;
    return DMU_OK;
}

extern "C" int dmu_phase_log(void *device_log, size_t records)
{
    clear_error();
    if ((device_log == nullptr) != (records == 0)) {
        set_error("dmu_phase_log: a log needs both a buffer and a record count (NULL and 0 turn it off)");
        return DMU_ERR_INVALID_ARG;
    }
    if ((uintptr_t)device_log % 8) {
        set_error("dmu_phase_log: the log is not 8-byte aligned");
        return DMU_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_phase_mu);
    g_phase_log = static_cast<uint64_t *>(device_log);
    g_phase_cap = records;
    g_phase_last = 0;
    g_phase_kind = 0;
    return DMU_OK;
}

extern "C" int dmu_phase_log_last(size_t *records, int *kind)
{
    clear_error();
    if (!records || !kind) {
        set_error("dmu_phase_log_last: NULL output");
        return DMU_ERR_INVALID_ARG;
    }
    std::lock_guard<std::mutex> lock(g_phase_mu);
    *records = g_phase_last;
    *kind = g_phase_kind;
    return DMU_OK;
}

extern "C" int dmu_device_info(int device, int *compute_units, int *max_clock_khz)
{
    clear_error();
    if (!compute_units || !max_clock_khz || device < 0) {
        set_error("dmu_device_info: NULL output or negative device");
        return DMU_ERR_INVALID_ARG;
    }
    int cu = 0, khz = 0;
    hipError_t e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device);
    if (e != hipSuccess) {
        set_error("dmu_device_info: %s", hipGetErrorString(e));
        return DMU_ERR_HIP;
    }
    *compute_units = cu;
    *max_clock_khz = khz;
    return DMU_OK;
}

extern "C" const char *dmu_status_string(int status)
{
    switch (status) {
    case DMU_OK: return "DMU_OK";
    case DMU_ERR_INVALID_ARG: return "DMU_ERR_INVALID_ARG: invalid argument";
    case DMU_ERR_UNSUPPORTED: return "DMU_ERR_UNSUPPORTED: unsupported type, variant or size";
    case DMU_ERR_HIP: return "DMU_ERR_HIP: HIP runtime error";
    default: return "unknown dmu status";
    }
}

extern "C" const char *dmu_last_error(void) { return g_err; }
