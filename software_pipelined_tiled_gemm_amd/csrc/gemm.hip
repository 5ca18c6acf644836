// C ABI of the software-pipelined tiled GEMM (declared in include/spgemm.h).
//
// Host side: argument validation (before any HIP call), the table of compiled
// tile configurations, the shape heuristic, the autotuner (the Pallas guide
// recommends autotuning max_concurrent_steps; the TileLang tutorial's chapter
// pairs pipelining with autotuning and bounds each candidate's shared memory by
// stages * (block_M + block_N) * block_K * bytes), and the launch.
#include "spgemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "errors.hpp"
#include "launch.hpp"

namespace spg {

namespace {
thread_local char g_last_hip_error[256] = "";
}  // namespace

gemm_status hip_fail(hipError_t e) {
    snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%d)", hipGetErrorString(e), (int)e);
    return GEMM_ERR_HIP;
}

const char* last_hip_error() { return g_last_hip_error; }

}  // namespace spg

// Count of the wave-specialized ring's bounded waits that gave up (each device holds
// its own copy of this word).  Kernels reach it through KArgs::wait_timeouts, the
// address hipGetSymbolAddress gives for the launching device.
static __device__ uint32_t g_wait_timeouts;

using spg::hip_fail;
using spg::KArgs;
using spg::launch_fn;
using spg::launch_pipelined;

namespace {

template <bool BF16, bool B_NK>
void launch_simple(const KArgs& a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((spg::simple_gemm<BF16, B_NK>), grid, dim3(256), 0, st, a);
}

struct Variant {
    gemm_tile_config cfg;
    launch_fn fn[2][2];  // [bf16][b_nk]
};

#define SPG_LP(BF, NK, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI) \
    launch_pipelined<BF, NK, BM, BN, BK, WM, WN, S, (SWZ != 0), LDM, PF, SCHED, (PERS != 0), MI>
#define SPG_ENTRY(BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI)                            \
    Variant{{BM, BN, BK, S, WM, WN, SWZ, 0, 1, LDM, PF, SCHED, PERS, 0, MI},                       \
            {{SPG_LP(false, false, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI),         \
              SPG_LP(false, true, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI)},         \
             {SPG_LP(true, false, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI),          \
              SPG_LP(true, true, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI)}}},
#ifdef SPG_POISON
// The poison library (a test build, see kPoison) holds only the units its build names
// with -DSPG_KEEP_<n>=~,1; the table lists the lines of those units.
#define SPG_CAT_(a, b) a##b
#define SPG_CAT(a, b) SPG_CAT_(a, b)
#define SPG_SECOND_(a, b, ...) b
#define SPG_SECOND(...) SPG_SECOND_(__VA_ARGS__)
#define SPG_KEPT(u) SPG_SECOND(SPG_CAT(SPG_KEEP_, u), 0)
#define SPG_VK_0(...)
#define SPG_VK_1(...) SPG_ENTRY(__VA_ARGS__)
#define SPG_V(unit, ...) SPG_CAT(SPG_VK_, SPG_KEPT(unit))(__VA_ARGS__)
#else
#define SPG_V(unit, ...) SPG_ENTRY(__VA_ARGS__)
#endif

const Variant kVariants[] = {
#include "variants.inc"
};
#undef SPG_V
#undef SPG_ENTRY
#undef SPG_LP
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
constexpr int kDefaultGroupM = 4;

struct ProblemKey {
    int64_t M, N, K;
    int in, out, bl, epi;
    bool operator<(const ProblemKey& o) const {
        return std::tie(M, N, K, in, out, bl, epi) < std::tie(o.M, o.N, o.K, o.in, o.out, o.bl, o.epi);
    }
};

std::mutex g_tuned_mu;
std::map<ProblemKey, gemm_tile_config> g_tuned;

bool same_tile(const gemm_tile_config& a, const gemm_tile_config& b) {
    return a.block_m == b.block_m && a.block_n == b.block_n && a.block_k == b.block_k &&
           a.stages == b.stages && a.wave_m == b.wave_m && a.wave_n == b.wave_n &&
           a.swizzle == b.swizzle && a.staging == b.staging && a.lookahead == b.lookahead &&
           a.schedule == b.schedule && a.persistent == b.persistent &&
           (a.mfma ? a.mfma : 32) == (b.mfma ? b.mfma : 32);
}

const Variant* find_variant(const gemm_tile_config& c) {
    for (const Variant& v : kVariants)
        if (same_tile(v.cfg, c)) return &v;
    return nullptr;
}

}  // namespace

struct gemm_plan {
    int64_t M, N, K;
    gemm_dtype in, out;
    gemm_b_layout bl;
    gemm_epilogue epi;
    bool simple;        // a shape the pipelined kernel does not take (K == 0, K < 8, ...)
    bool rows_aligned;  // every row of A and B starts 16 bytes after the previous one
    const Variant* var;     // the configuration gemm_run launches for 16-byte aligned A and B
    gemm_tile_config cfg;
    const Variant* uvar;    // its misaligned-operand twin (copy mode 7): A or B not 16-byte
    gemm_tile_config ucfg;  // aligned at run time (the same as var when the rows are not)
};

namespace {

bool valid_dtype_in(int d) { return d == GEMM_F16 || d == GEMM_BF16; }
bool valid_dtype_out(int d) { return d == GEMM_F16 || d == GEMM_BF16 || d == GEMM_F32; }

// Shape conditions of the pipelined kernel: 32-bit buffer offsets, and rows long
// enough to hold one 8-element copy window.  A copy resource spans at most 256 rows of
// A (or of a [N,K] B) or all of a [K,N] B, plus up to 63 k of the leading partial
// k-tile; it must stay within 2^31 bytes so that the out-of-range offset 2^31 reads
// zero.  A K-contiguous row (A, B stored [N,K]) must hold 8 elements (K >= 8), and so
// must a row of B stored [K,N] (N >= 8): copy mode 7 loads a chunk that straddles the
// edge of the valid range from the 8-element window inside the row.  Anything else
// (K == 0 included, which writes epi(0)) runs on the simple kernel.
bool pipelined_fits(int64_t M, int64_t N, int64_t K, gemm_b_layout bl) {
    if (K <= 0 || M <= 0 || N <= 0) return false;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return false;
    if (K < 8) return false;
    const int64_t lim = (int64_t)1 << 31;
    if (256 * (K + 64) * 2 > lim) return false;
    if (bl == GEMM_B_KN) {
        if (N < 8) return false;
        if ((K + 64) * N * 2 > lim) return false;
    }
    return true;
}

// Rows of A and B 16 bytes apart: the direct-to-LDS copy modes need this (and 16-byte
// aligned base pointers, checked at launch); otherwise copy mode 7 runs.
bool rows_aligned(int64_t N, int64_t K, gemm_b_layout bl) {
    return K % 8 == 0 && (bl == GEMM_B_NK || N % 8 == 0);
}

const Variant* find_cfg(int bm, int bn, int bk, int stages, int staging, int wm, int wn,
                        int persistent = 0, int mfma = 32, int schedule = 0) {
    for (const Variant& v : kVariants)
        if (v.cfg.block_m == bm && v.cfg.block_n == bn && v.cfg.block_k == bk &&
            v.cfg.stages == stages && v.cfg.staging == staging && v.cfg.swizzle == 1 &&
            v.cfg.wave_m == wm && v.cfg.wave_n == wn && v.cfg.lookahead == 1 &&
            v.cfg.schedule == schedule && v.cfg.persistent == persistent && v.cfg.mfma == mfma)
            return &v;
    return nullptr;
}

// Compute units of the current device (cached per device; 0 if the query fails).
int cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 0;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    return n;
}

// Device address of g_wait_timeouts on the current device (resolved once per device;
// nullptr if there is no device or the lookup fails).
uint32_t* wait_word() {
    static uint32_t* cache[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    uint32_t* p = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
    if (p) return p;
    if (hipGetSymbolAddress((void**)&p, HIP_SYMBOL(g_wait_timeouts)) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    __atomic_store_n(&cache[dev], p, __ATOMIC_RELEASE);
    return p;
}

gemm_tile_config heuristic(int64_t M, int64_t N, int64_t K, gemm_b_layout bl, bool aligned) {
    // Estimated time of a candidate = rounds of the device's CUs it needs x its tile's
    // area / its measured per-tile throughput relative to 256x256 (bf16 NN 8192^3
    // and the 1024x8192x8192 shard on MI355X: 256x128 runs at 0.91 of the 256x256
    // rate per output, 128x128 at 0.77 (8 waves of 16x16x32; 925 against 709 us at
    // 8192^3), 192x256 at 0.80 (3072x4096x4096) to 0.88 (6144x8192x8192: 4 rounds of
    // 192x256 against 3 of 256x256, 623 vs 549 us)).
    // The smallest estimate wins: 256x256 as long as the grid is not much less than
    // one round, 192x256 where its rows fill the CUs better (M = 3072: 16 x 16 tiles
    // against 12 x 16), 256x128 for half-size grids, 128x128 for small problems.
    // Every tile runs 8 waves of 16x16x32 MFMAs (measured against 32x32x16 with the
    // same tile, interleaved in one process, +2..9% on every benchmark shape of the
    // large tiles; 128x128 with 8 waves of 32x64 against 4 waves of 64x64 of 32x32x16:
    // -10..-26% time on 256^3 .. 2048^3 and 1024x2048x4096).
    const int cc = cu_count();
    const int64_t cus = cc > 0 ? cc : 256;   // 256 on MI355X; also the planning default without a device
    struct Cand { int bm, bn, bk, st, wm, wn, mfma; double eff; };
    const Cand cands[] = {{256, 256, 64, 2, 128, 64, 16, 1.0},
                          {192, 256, 64, 2, 96, 64, 16, 0.85},
                          {256, 128, 64, 3, 64, 64, 16, 0.91},
                          {128, 128, 64, 3, 32, 64, 16, 0.77}};
    // Misaligned operands (copy mode 7, register-staged, 32x32x16): the same cost model
    // over the tiles compiled for that mode
    const Cand ucands[] = {{256, 256, 64, 2, 128, 64, 32, 1.0},
                           {256, 128, 64, 3, 128, 64, 32, 0.85},
                           {128, 128, 64, 3, 64, 64, 32, 0.66}};
    // Only candidates the library holds compete (a build may compile a subset of
    // variants.inc); with none, the zero configuration returned matches no variant.
    if (!aligned) {
        const Variant* ub = nullptr;
        double ub_t = 0.0;
        for (const Cand& c : ucands) {
            const Variant* v = find_cfg(c.bm, c.bn, c.bk, c.st, 7, c.wm, c.wn, 0, c.mfma);
            if (!v) continue;
            const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
            const double t = (double)((tiles + cus - 1) / cus) * c.bm * c.bn / c.eff;
            if (!ub || t < ub_t) { ub = v; ub_t = t; }
        }
        if (!ub) return gemm_tile_config{};
        gemm_tile_config c = ub->cfg;
        c.group_m = kDefaultGroupM;
        c.xcd_remap = 1;
        return c;
    }
    const Cand* best = nullptr;
    double best_t = 0.0;
    for (const Cand& c : cands) {
        if (!find_cfg(c.bm, c.bn, c.bk, c.st, 0, c.wm, c.wn, 0, c.mfma)) continue;
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        const double t = (double)((tiles + cus - 1) / cus) * c.bm * c.bn / c.eff;
        if (!best || t < best_t) { best = &c; best_t = t; }
    }
    if (!best) return gemm_tile_config{};
    // Grids of two rounds or more on the 256x256 tile: the B-deep ring (staging 6, three
    // B slots).  With B stored [K,N] under the compiler-placed schedule: a [K,N] k-tile
    // of B is 64 rows 2*N bytes apart, and its copies are the ones that land late
    // (measured interleaved at 8192^3, bf16 NN 710.0 -> 701.3 us, fp16 NN 753.6 ->
    // 747.5 us).  With B stored [N,K] under the ping-pong schedule, which is 2-3% ahead
    // of the two-slot hand-placed ring there in bf16 and ~1% in fp16, but ~2% behind the
    // compiler-placed B-deep ring with B stored [K,N].  Grids of one round keep the
    // two-slot ring (the ping-pong schedule is even there).
    const int64_t tiles = ((M + best->bm - 1) / best->bm) * ((N + best->bn - 1) / best->bn);
    const Variant* v = nullptr;
    if (best->bm == 256 && best->bn == 256 && tiles >= 2 * cus)
        v = find_cfg(256, 256, 64, 2, 6, best->wm, best->wn, 0, 16, bl == GEMM_B_KN ? 1 : 2);
    // 128x128: S = 3 (96 KiB: one workgroup per CU) on grids of less than two rounds
    // with more than 16 k-tiles or at least half a round of tiles, else S = 2 (64 KiB:
    // two workgroups can share a CU).  On a grid of about one round, S = 2 lets the
    // dispatcher put two workgroups on one CU, which then sets the kernel time.
    // Measured: 1024x2048x4096 (128 tiles) 24.9 us with S = 3 against 39.6 with S = 2,
    // 2048^3 19.3 against 23.4, 2048x2048x1024 (256 tiles, 16 k-tiles) 14.4 against
    // 14.4 .. 16.2 from run to run; but 256^3 4.4 against 5.1 us, 1024^3 (64 tiles) 8.7
    // against 9.5, 2048x4096x4096 (512 tiles) 65.7 against 70.6, 8192^3 925 against 958.
    int st = best->st;
    const int64_t nk = (K + best->bk - 1) / best->bk;
    if (best->bm == 128 && best->bn == 128)
        st = (tiles < 2 * cus && (nk > 16 || 2 * tiles >= cus)) ? 3 : 2;
    // Schedule of the two-slot / three-slot rings: compiler-placed (with its interleaving
    // hint) for 256x128 and for 256x256 with more than 16 k-tiles, hand-placed otherwise.
    // Measured interleaved against the hand-placed schedule with a control copy:
    // 1024x8192x8192 (256x128) bf16 NN -2.6%, fp16 TN -1.3%; 4096^3 (256x256, one round)
    // fp16 TN -2.1%, bf16 NN -1.3%; but 3000x5000x1000 (16 k-tiles) +0.8%, 192x256 even,
    // and the 128x128 tile +0.5 .. +6% (2048^3).
    int sched = 0;
    if ((best->bm == 256 && best->bn == 128) || (best->bm == 256 && best->bn == 256 && nk > 16))
        sched = 1;
    if (!v) v = find_cfg(best->bm, best->bn, best->bk, st, 0, best->wm, best->wn, 0, best->mfma, sched);
    // (the candidate's own two-slot / three-slot ring, compiled: checked above)
    if (!v) v = find_cfg(best->bm, best->bn, best->bk, best->st, 0, best->wm, best->wn, 0, best->mfma);
    gemm_tile_config c = v->cfg;
    // 4 tile rows per raster group: with the 16x16x32 tiles at 8192^3 (32 tile rows),
    // measured interleaved: group_m 2 / 4 / 8 / 16 / 32 = 758 / 730 / 740 / 752 / 911 us
    // (NN) and 765 / 733 /741 / 766 / 934 us (TN); the 32x32x16 kernel preferred 8
    c.group_m = kDefaultGroupM;
    c.xcd_remap = 1;
    return c;
}

// Largest power of two (at most 16) dividing an address.
int32_t alignment_of(const void* p) {
    const uintptr_t v = (uintptr_t)p;
    for (int32_t a = 16; a > 1; a >>= 1)
        if (v % (uintptr_t)a == 0) return a;
    return 1;
}

KArgs make_args(const gemm_plan* p, const void* A, const void* B, void* C, int bm, int bn) {
    KArgs a;
    a.A = (const uint16_t*)A;
    a.B = (const uint16_t*)B;
    a.C = C;
    a.M = (int32_t)p->M;
    a.N = (int32_t)p->N;
    a.K = (int32_t)p->K;
    a.tiles_m = (int32_t)((p->M + bm - 1) / bm);
    a.tiles_n = (int32_t)((p->N + bn - 1) / bn);
    a.group_m = p->cfg.group_m > 0 ? p->cfg.group_m : kDefaultGroupM;
    a.xcd_remap = p->cfg.xcd_remap ? 1 : 0;
    a.out_dtype = (int32_t)p->out;
    a.epilogue = (int32_t)p->epi;
    a.persistent = 0;
    a.store_direct = p->cfg.store ? 1 : 0;
    a.wait_timeouts = wait_word();
    a.c_align = alignment_of(C);
    return a;
}

// Shapes the persistent kernel takes: every k-tile whole (K % block_k == 0), a
// 16-bit output (its epilogue staging holds 2-byte values) and, for B stored
// [K,N], whole column tiles (its copies carry no column masks).
bool persistent_fits(const gemm_plan* p, const gemm_tile_config& c) {
    if (!c.persistent || c.block_k <= 0 || c.block_n <= 0) return false;
    if (p->out == GEMM_F32 || p->K % c.block_k != 0) return false;
    if (p->bl == GEMM_B_KN && p->N % c.block_n != 0) return false;
    return true;
}

// The configuration a launch with these operand pointers runs: the simple kernel
// (nullptr), `var`, or, when A or B is not 16-byte aligned and `var` copies straight
// to LDS, the plan's misaligned-operand twin.  (C's alignment only selects 16-byte or
// element stores inside the epilogue.)
const Variant* pick(const gemm_plan* p, const gemm_tile_config& cfg, const Variant* var,
                    const void* A, const void* B, gemm_tile_config* used) {
    if (p->simple || var == nullptr) return nullptr;
    const bool ab16 = ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0);
    if (cfg.staging != 7 && !ab16) {
        *used = p->ucfg;
        used->group_m = cfg.group_m;
        used->xcd_remap = cfg.xcd_remap;
        return p->uvar;
    }
    *used = cfg;
    return var;
}

gemm_status launch_plan(const gemm_plan* p, const gemm_tile_config& cfg_in, const Variant* var_in,
                        const void* A, const void* B, void* C, hipStream_t st) {
    const bool bf = p->in == GEMM_BF16;
    const bool nk = p->bl == GEMM_B_NK;
    gemm_tile_config cfg = cfg_in;
    const Variant* var = pick(p, cfg_in, var_in, A, B, &cfg);
    if (var == nullptr) {
        gemm_plan q = *p;
        q.cfg.group_m = 1;
        KArgs a = make_args(&q, A, B, C, 64, 64);
        dim3 grid((unsigned)a.tiles_n, (unsigned)a.tiles_m);
        (bf ? (nk ? launch_simple<true, true> : launch_simple<true, false>)
            : (nk ? launch_simple<false, true> : launch_simple<false, false>))(a, grid, st);
    } else {
        gemm_plan q = *p;
        q.cfg = cfg;
        KArgs a = make_args(&q, A, B, C, cfg.block_m, cfg.block_n);
        int64_t wgs = (int64_t)a.tiles_m * a.tiles_n;
        if (persistent_fits(p, cfg) && !cfg.store) {
            // one workgroup per CU (its LDS allows no second), each walking its tiles
            const int cus = cu_count();
            if (cus > 0) {
                a.persistent = 1;
                wgs = std::min<int64_t>(wgs, cus);
            }
        }
        dim3 grid((unsigned)wgs);
        var->fn[bf ? 1 : 0][nk ? 1 : 0](a, grid, st);
    }
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? GEMM_OK : hip_fail(e);
}

}  // namespace

extern "C" {

const char* gemm_status_string(gemm_status s) {
    switch (s) {
        case GEMM_OK: return "ok";
        case GEMM_ERR_INVALID_ARG: return "invalid argument";
        case GEMM_ERR_UNSUPPORTED: return "unsupported";
        case GEMM_ERR_OUT_OF_MEMORY: return "out of memory";
        case GEMM_ERR_HIP: return "HIP runtime error";
        case GEMM_ERR_INTERNAL: return "internal error";
    }
    return "unknown status";
}

const char* gemm_last_hip_error(void) { return spg::last_hip_error(); }

gemm_status gemm_wait_timeouts(uint32_t* count, int32_t reset) {
    if (!count) return GEMM_ERR_INVALID_ARG;
    *count = 0;
    uint32_t* p = wait_word();
    if (!p) {
        int n = 0;
        const hipError_t e = hipGetDeviceCount(&n);
        return hip_fail(e != hipSuccess ? e : hipErrorNoDevice);
    }
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(count, p, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess && reset) e = hipMemset(p, 0, sizeof(uint32_t));
    if (e == hipSuccess && reset) e = hipDeviceSynchronize();
    return e == hipSuccess ? GEMM_OK : hip_fail(e);
}

int32_t gemm_num_configs(void) { return kNumVariants; }

gemm_status gemm_list_config(int32_t index, gemm_tile_config* out) {
    if (!out || index < 0 || index >= kNumVariants) return GEMM_ERR_INVALID_ARG;
    *out = kVariants[index].cfg;
    out->group_m = kDefaultGroupM;
    return GEMM_OK;
}

int64_t gemm_lds_bytes(const gemm_tile_config* c) {
    if (!c) return -1;
    const int64_t ring = (int64_t)c->stages * ((int64_t)c->block_m + c->block_n) * c->block_k * 2;
    // the A-deep ring holds one more k-tile of A, the B-deep ring one more of B
    if (c->staging == 4) return ring + (int64_t)c->block_m * c->block_k * 2;
    if (c->staging == 6) return ring + (int64_t)c->block_n * c->block_k * 2;
    return ring;
}

gemm_status gemm_create(gemm_handle* out, int64_t M, int64_t N, int64_t K, gemm_dtype in_dtype,
                        gemm_dtype out_dtype, gemm_b_layout b_layout, gemm_epilogue epilogue,
                        const gemm_tile_config* force) {
    if (!out) return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return GEMM_ERR_UNSUPPORTED;
    if (!valid_dtype_in((int)in_dtype) || !valid_dtype_out((int)out_dtype)) return GEMM_ERR_INVALID_ARG;
    if (b_layout != GEMM_B_KN && b_layout != GEMM_B_NK) return GEMM_ERR_INVALID_ARG;
    if (epilogue != GEMM_EPI_NONE && epilogue != GEMM_EPI_GELU_TANH && epilogue != GEMM_EPI_RELU)
        return GEMM_ERR_INVALID_ARG;

    const Variant* var = nullptr;
    gemm_tile_config cfg;
    if (force) {
        if (force->block_m <= 0 || force->block_n <= 0 || force->block_k <= 0 ||
            force->stages <= 0 || force->wave_m <= 0 || force->wave_n <= 0 ||
            force->group_m < 0 || (force->swizzle != 0 && force->swizzle != 1) ||
            (force->xcd_remap != 0 && force->xcd_remap != 1) ||
            force->staging < 0 || force->staging > 7 ||
            (force->store != 0 && force->store != 1) ||
            (force->mfma != 0 && force->mfma != 16 && force->mfma != 32) ||
            (force->lookahead != 1 && force->lookahead != 2) ||
            force->schedule < 0 || force->schedule > 2 ||
            (force->persistent != 0 && force->persistent != 1))
            return GEMM_ERR_INVALID_ARG;
        if (gemm_lds_bytes(force) > 160 * 1024) return GEMM_ERR_UNSUPPORTED;
        var = find_variant(*force);
        if (!var) return GEMM_ERR_UNSUPPORTED;
        cfg = *force;
        if (cfg.group_m == 0) cfg.group_m = kDefaultGroupM;
        if (cfg.mfma == 0) cfg.mfma = 32;
    } else {
        bool have = false;
        {
            std::lock_guard<std::mutex> lk(g_tuned_mu);
            auto it = g_tuned.find(ProblemKey{M, N, K, in_dtype, out_dtype, b_layout, epilogue});
            if (it != g_tuned.end()) {
                cfg = it->second;
                have = true;
            }
        }
        if (!have) cfg = heuristic(M, N, K, b_layout, rows_aligned(N, K, b_layout));
        var = find_variant(cfg);
        if (!var) return GEMM_ERR_INTERNAL;
    }
    // rows that are not 16 bytes apart only go through copy mode 7
    const bool ra = rows_aligned(N, K, b_layout);
    if (!ra && cfg.staging != 7 && pipelined_fits(M, N, K, b_layout)) return GEMM_ERR_UNSUPPORTED;
    gemm_tile_config ucfg = cfg;
    const Variant* uvar = var;
    if (cfg.staging != 7) {
        // (a library without copy mode 7 plans no twin: misaligned pointers then take the
        // simple kernel)
        ucfg = heuristic(M, N, K, b_layout, false);
        uvar = find_variant(ucfg);
    }
    gemm_plan* p = new (std::nothrow) gemm_plan;
    if (!p) return GEMM_ERR_OUT_OF_MEMORY;
    p->M = M;
    p->N = N;
    p->K = K;
    p->in = in_dtype;
    p->out = out_dtype;
    p->bl = b_layout;
    p->epi = epilogue;
    p->simple = !pipelined_fits(M, N, K, b_layout);
    p->rows_aligned = ra;
    p->var = var;
    p->cfg = cfg;
    p->uvar = uvar;
    p->ucfg = ucfg;
    (void)wait_word();   // resolve the device's error word now, outside any graph capture
    *out = p;
    return GEMM_OK;
}

gemm_status gemm_destroy(gemm_handle h) {
    delete h;
    return GEMM_OK;
}

gemm_status gemm_get_config(gemm_handle h, gemm_tile_config* out) {
    if (!h || !out) return GEMM_ERR_INVALID_ARG;
    *out = h->cfg;
    if (h->simple) {
        *out = gemm_tile_config{64, 64, 0, 1, 64, 64, 0, 1, 0, 0};
    }
    return GEMM_OK;
}

gemm_status gemm_launch_config(gemm_handle h, const void* A, const void* B, const void* C,
                               gemm_tile_config* out) {
    if (!h || !out) return GEMM_ERR_INVALID_ARG;
    (void)C;
    gemm_tile_config used = h->cfg;
    if (pick(h, h->cfg, h->var, A, B, &used) == nullptr)
        used = gemm_tile_config{64, 64, 0, 1, 64, 64, 0, 1, 0, 0};
    *out = used;
    return GEMM_OK;
}

gemm_status gemm_run(gemm_handle h, const void* A, const void* B, void* C, hipStream_t stream) {
    if (!h) return GEMM_ERR_INVALID_ARG;
    if (h->M == 0 || h->N == 0) return GEMM_OK;
    if (!C) return GEMM_ERR_INVALID_ARG;
    if (h->K > 0 && (!A || !B)) return GEMM_ERR_INVALID_ARG;
    return launch_plan(h, h->cfg, h->var, A, B, C, stream);
}

gemm_status gemm_autotune(gemm_handle h, const void* A, const void* B, void* C,
                          hipStream_t stream, int reps, double* best_us) {
    if (!h || reps <= 0) return GEMM_ERR_INVALID_ARG;
    if (h->M == 0 || h->N == 0) return GEMM_OK;
    if (!C || (h->K > 0 && (!A || !B))) return GEMM_ERR_INVALID_ARG;
    if (h->simple) {
        if (best_us) *best_us = -1.0;
        return GEMM_OK;
    }
    hipEvent_t e0, e1;
    hipError_t he = hipEventCreate(&e0);
    if (he != hipSuccess) return hip_fail(he);
    he = hipEventCreate(&e1);
    if (he != hipSuccess) {
        (void)hipEventDestroy(e0);
        return hip_fail(he);
    }
    gemm_status st = GEMM_OK;
    float best = -1.0f;
    gemm_tile_config best_cfg = h->cfg;
    const Variant* best_var = h->var;
    const int groups[] = {4, 8, 16};
    const bool need7 = !h->rows_aligned || (uintptr_t)A % 16 != 0 || (uintptr_t)B % 16 != 0;
    for (const Variant& v : kVariants) {
        if (v.cfg.swizzle == 0 || v.cfg.stages == 1) continue;  // ablations are not candidates
        if (need7 && v.cfg.staging != 7) continue;              // direct copies need aligned rows
        for (int g : groups) {
            gemm_tile_config c = v.cfg;
            c.group_m = g;
            c.xcd_remap = 1;
            st = launch_plan(h, c, &v, A, B, C, stream);  // warm-up
            if (st != GEMM_OK) break;
            if ((he = hipEventRecord(e0, stream)) != hipSuccess) { st = hip_fail(he); break; }
            for (int r = 0; r < reps && st == GEMM_OK; ++r) st = launch_plan(h, c, &v, A, B, C, stream);
            if (st != GEMM_OK) break;
            if ((he = hipEventRecord(e1, stream)) != hipSuccess) { st = hip_fail(he); break; }
            if ((he = hipEventSynchronize(e1)) != hipSuccess) { st = hip_fail(he); break; }
            float ms = 0.0f;
            if ((he = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) { st = hip_fail(he); break; }
            if (best < 0.0f || ms < best) {
                best = ms;
                best_cfg = c;
                best_var = &v;
            }
        }
        if (st != GEMM_OK) break;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (st != GEMM_OK) return st;
    h->cfg = best_cfg;
    h->var = best_var;
    {
        std::lock_guard<std::mutex> lk(g_tuned_mu);
        g_tuned[ProblemKey{h->M, h->N, h->K, h->in, h->out, h->bl, h->epi}] = best_cfg;
    }
    if (best_us) *best_us = best > 0 ? 1000.0 * best / reps : -1.0;
    return GEMM_OK;
}

}  // extern "C"
