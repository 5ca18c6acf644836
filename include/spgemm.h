/*
 * spgemm.h -- C ABI of the software-pipelined, tiled MFMA GEMM for MI355X (gfx950).
 *
 *   C[M,N] = epi( A[M,K] . B )       fp16 or bf16 inputs, fp32 accumulation,
 *                                    fp16 / bf16 / fp32 output.
 *
 * The operation is the output-stationary tiled matrix product that the Mosaic
 * GPU pipelining guide (Pallas) builds in "Example: matmul kernel on Hopper
 * GPUs" ([M,K] @ [K,N], each output block owned by one program, K reduced by a
 * pipelined sequential loop) and that the TileLang pipelined GEMM tutorial
 * (chapter "pipeline and autotuning", matmul_auto) writes with B stored [N,K]
 * and transpose_B=True.  The optional epilogue is the tanh approximation of
 * GELU that the XLA:GPU emitters page fuses in its loop-emitter example and the
 * Triton lecture notes write in their GeLU kernel:
 *     gelu(x) = 0.5 x (1 + tanh(0.7978845608 (x + 0.044715 x^3))),
 * applied to the fp32 accumulator before the output conversion.
 *
 * Conventions shared by every entry point:
 *   - Matrices are dense and row-major.  A is [M,K] (leading dimension K).
 *     B is [K,N] (GEMM_B_KN, leading dimension N) or [N,K] (GEMM_B_NK,
 *     leading dimension K).  C is [M,N] (leading dimension N).
 *   - A, B and C are device pointers owned by the caller; the library never
 *     frees or retains them.  C must not overlap A or B (not checked).  Any 2-byte
 *     aligned pointer is accepted (4-byte for an fp32 C).  When the rows of A and B
 *     are 16 bytes apart (K % 8 == 0, and N % 8 == 0 for B stored [K,N]) and A and
 *     B are 16-byte aligned, k-tiles are copied straight from memory into LDS;
 *     otherwise the same MFMA kernel stages them through registers with 16-byte
 *     loads at any 2-byte alignment (copy mode 7 below).  A C that is not 16-byte
 *     aligned is written with element stores.
 *   - Out-of-range elements of partial tiles contribute exactly zero and are
 *     never written: any M, N, K >= 0 is accepted (the masked tails of the Triton
 *     lecture notes' matmul, other = 0).  M == 0 or N == 0 is a no-op; K == 0
 *     writes epi(0) = 0 everywhere.  K < 8, N < 8 with B stored [K,N], and
 *     operands whose copy windows would exceed 2^31 bytes run a simple
 *     bounds-checked kernel.
 *   - Errors are reported only through gemm_status; nothing aborts and no C++
 *     exception crosses this interface.  Argument checks run before any HIP
 *     call, so they behave the same on a machine without a GPU.
 *   - Rounding to fp16/bf16 is to nearest, ties to even.
 */
#ifndef SPGEMM_H
#define SPGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = 1,   /* NULL handle/pointer, negative size, unknown enum, bad config */
    GEMM_ERR_UNSUPPORTED = 2,   /* valid request this build cannot run (e.g. forced tile unknown) */
    GEMM_ERR_OUT_OF_MEMORY = 3, /* host or device allocation failed */
    GEMM_ERR_HIP = 4,           /* a HIP runtime call failed (no device, launch error, ...) */
    GEMM_ERR_INTERNAL = 5
} gemm_status;

typedef enum { GEMM_F16 = 0, GEMM_BF16 = 1, GEMM_F32 = 2 /* output only */ } gemm_dtype;

typedef enum {
    GEMM_B_KN = 0, /* B row-major [K,N]  ("NN") */
    GEMM_B_NK = 1  /* B row-major [N,K]  ("TN", transpose_B) */
} gemm_b_layout;

/* Epilogue applied to the fp32 accumulator before the output conversion:
 *   GEMM_EPI_GELU_TANH  the tanh approximation of GELU above;
 *   GEMM_EPI_RELU       max(x, 0), what the Triton lecture notes' matmul kernel
 *                       (Matmul section, matmul_relu_kernel) applies to its
 *                       accumulator before the store; -0 becomes +0. */
typedef enum { GEMM_EPI_NONE = 0, GEMM_EPI_GELU_TANH = 1, GEMM_EPI_RELU = 2 } gemm_epilogue;

/* Tile configuration of the pipelined kernel.
 *   block_m x block_n   output tile of one workgroup (128, 192 or 256 rows; 128 or
 *                       256 columns; gemm_list_configs() lists the compiled ones)
 *   block_k             K extent of one pipeline stage (32 or 64)
 *   stages              LDS ring depth S (1 = no overlap, the serial K loop of the
 *                       TileLang tutorial's matmul_plain; 2..4 = loads of k-tile t+S-1
 *                       in flight while k-tile t is multiplied)
 *   wave_m x wave_n     output tile of one 64-lane wave (multiples of 32)
 *   swizzle             1 = XOR-swizzled LDS layout, 0 = plain row layout (ablation)
 *   group_m             tile-raster group height in tiles (L2 reuse); 0 = default (4)
 *   xcd_remap           1 = give each of the 8 XCDs a contiguous range of tiles
 *   staging             0 = k-tiles are copied straight from memory into LDS
 *                       (buffer_load ... lds), a k-tile's copies issued in the
 *                       first stage after the barrier that frees their slot (one per
 *                       MFMA step, or one every second step where the stage has at
 *                       least twice as many MFMAs as copies);
 *                       1 = copied into VGPRs one k-tile ahead and written to LDS
 *                       with ds_write_b128; 2 = straight into LDS, the copies of a
 *                       k-tile spread evenly between two barriers (stages >= 3);
 *                       3 = wave-specialized (the Pallas guide's warp-specialized
 *                       pipeline): one producer wave issues every copy, the
 *                       consumer waves only read LDS and multiply, and per-slot
 *                       counters in LDS replace the barrier;
 *                       4 = as 0, with A in a ring one slot deeper than B (stages =
 *                       2: three A slots, two B slots), so the copies of A have two
 *                       k-tiles to land and those of B one;
 *                       6 = as 4 with the roles swapped: B in a ring one slot
 *                       deeper than A (stages = 2: two A slots, three B slots);
 *                       compiled with schedule = 1 and 2 (16x16x32 tiles);
 *                       5 = as 0, with a slot refilled one k-tile after its release
 *                       (the Pallas guide's release delay of 1; stages >= 3): S-1
 *                       k-tiles in flight instead of S;
 *                       7 = as 1, for operands whose rows or base pointers are not
 *                       16-byte aligned: 16-byte loads at any 2-byte alignment, the
 *                       chunk that straddles k = 0 (first k-tile) or column N (B
 *                       stored [K,N]) loaded from the 8-element window inside the
 *                       valid range and shifted into place in registers, its
 *                       out-of-range elements zeroed.  gemm_create plans it when
 *                       K % 8 != 0 or (B stored [K,N]) N % 8 != 0, and gemm_run
 *                       switches to it when A or B is not 16-byte aligned
 *   lookahead           MFMA k-steps between the LDS read of an operand fragment and
 *                       its use: 1 (two fragment sets in registers) or 2 (four sets;
 *                       block_k 64, stages >= 2)
 *   schedule            0 = instructions of a stage placed by hand (each MFMA step
 *                       followed by its copy op and LDS reads, the TileLang
 *                       tutorial's manual stage/order placement); 1 = the same
 *                       instructions placed by the compiler (its planned pipeline);
 *                       2 = ping-pong (staging 6, 8 waves of 16x16x32 only): the two
 *                       waves of each SIMD take turns, one issuing a k-step's MFMAs
 *                       while the other reads the next fragments and copies, with a
 *                       workgroup barrier between turns (a schedule of this library,
 *                       not of the pages)
 *   persistent          1 = one workgroup per compute unit, each computing the tiles
 *                       g, g + G, g + 2G, ... (G = workgroups) as one continuous
 *                       pipeline of k-tiles, so the copies of a tile's first k-tiles
 *                       overlap the previous tile's last ones and its epilogue (an
 *                       extension of this library: the pages pipeline the K loop of
 *                       one output block); the epilogue stages through a further
 *                       32 x wave_n x 2 bytes of LDS per wave.  Used only when
 *                       K % block_k == 0, the output is fp16/bf16 and, for GEMM_B_KN,
 *                       N % block_n == 0; other problems run the same tile with one
 *                       workgroup per tile.  0 = one workgroup per tile.
 *   store               0 = the epilogue stages each wave's output through LDS and
 *                       writes 16-byte row segments (default); 1 = for fp16/bf16
 *                       output, each lane stores its own accumulator values straight
 *                       from registers (4 consecutive outputs per store; the ablation
 *                       of the staging).  fp32 output and the persistent and
 *                       wave-specialized modes always stage.
 *   mfma                32 (or 0) = v_mfma_f32_32x32x16 tiles; 16 = v_mfma_f32_16x16x32
 *                       tiles (block_k 64, lookahead 1, not persistent): the same
 *                       flops with half the accumulator register traffic per flop
 * The LDS a configuration needs is stages * (block_m + block_n) * block_k * 2 bytes
 * (the shared-memory bound of the TileLang tutorial's shared_bytes()), plus
 * block_m * block_k * 2 for staging 4 or block_n * block_k * 2 for staging 6, at
 * most 160 KiB. */
typedef struct {
    int32_t block_m, block_n, block_k;
    int32_t stages;
    int32_t wave_m, wave_n;
    int32_t swizzle;
    int32_t group_m;
    int32_t xcd_remap;
    int32_t staging;
    int32_t lookahead;
    int32_t schedule;
    int32_t persistent;
    int32_t store;
    int32_t mfma;
} gemm_tile_config;

typedef struct gemm_plan* gemm_handle;

/* Create a plan for one problem.  `force` == NULL picks a configuration from the
 * shape (or the best one a previous gemm_autotune found for the same problem in
 * this process); otherwise the forced configuration is used and must be one of
 * gemm_list_configs() (group_m / xcd_remap may take any value >= 0 / {0,1}).
 * Allocates host memory only; never synchronizes.
 * Errors: INVALID_ARG (out NULL, M/N/K < 0, unknown dtype/layout/epilogue,
 * in_dtype F32, malformed force), UNSUPPORTED (force not compiled in). */
gemm_status gemm_create(gemm_handle* out, int64_t M, int64_t N, int64_t K, gemm_dtype in_dtype,
                        gemm_dtype out_dtype, gemm_b_layout b_layout, gemm_epilogue epilogue,
                        const gemm_tile_config* force);

/* Enqueue C = epi(A . B) on `stream` (0 = null stream).  Asynchronous: no
 * allocation, no synchronization, exactly one kernel launch, so it may be captured
 * into a HIP graph (the pointers are baked into the captured launch).  A, B, C are
 * device pointers as described above.  Errors: INVALID_ARG (NULL handle, or NULL
 * pointer with a non-empty operand), HIP (launch failure). */
gemm_status gemm_run(gemm_handle h, const void* A, const void* B, void* C, hipStream_t stream);

/* Release a plan.  NULL is a no-op. */
gemm_status gemm_destroy(gemm_handle h);

/* The configuration a plan launches for 16-byte aligned A and B (copy mode 7 when
 * the rows themselves are not 16 bytes apart); a plan on the simple kernel reports
 * block_k = 0. */
gemm_status gemm_get_config(gemm_handle h, gemm_tile_config* out);

/* The configuration gemm_run would launch with these operand pointers: as
 * gemm_get_config, except that an A or B that is not 16-byte aligned selects the
 * plan's copy-mode-7 configuration.  No HIP call.  Errors: INVALID_ARG (NULL h or
 * out). */
gemm_status gemm_launch_config(gemm_handle h, const void* A, const void* B, const void* C,
                               gemm_tile_config* out);

/* Time every compiled configuration that fits the plan's problem on the caller's
 * buffers, `reps` launches each after one warm-up, and make the fastest the plan's
 * configuration; also remembered for later gemm_create calls with the same problem in
 * this process.  C is overwritten: on return it holds the product as the last
 * configuration timed computed it (within the same tolerance).  Synchronizes `stream`.
 * best_us (may be NULL) receives the winner's mean time per launch in microseconds. */
gemm_status gemm_autotune(gemm_handle h, const void* A, const void* B, void* C,
                          hipStream_t stream, int reps, double* best_us);

/* Static table of compiled configurations (valid for any dtype/layout). */
int32_t gemm_num_configs(void);
gemm_status gemm_list_config(int32_t index, gemm_tile_config* out);

/* LDS bytes a configuration needs: stages * (block_m + block_n) * block_k * 2, plus
 * block_m * block_k * 2 for staging 4 or block_n * block_k * 2 for staging 6.
 * Returns -1 for a NULL cfg. */
int64_t gemm_lds_bytes(const gemm_tile_config* cfg);

/* Bounded waits of the wave-specialized ring (staging 3, the Pallas guide's
 * warp-specialized pipeline with "consumed" counters) that gave up on the current
 * device since the library was loaded or since the last reset.  Each wait on an LDS
 * counter polls for about 0.1 s and then lets the wave go on instead of hanging; a
 * give-up therefore means some launch produced a wrong C, and it is counted in a device
 * word that this call reads back.  Waits for the device to finish all its work first;
 * reset != 0 then clears the word.  *count receives the number (0 on error).
 * Errors: INVALID_ARG (count NULL), HIP (no device, or a HIP call failed). */
gemm_status gemm_wait_timeouts(uint32_t* count, int32_t reset);

/* Human-readable name of a status code (static storage). */
const char* gemm_status_string(gemm_status s);

/* Text of the last HIP error this thread's calls into the library saw (hipGetErrorString
 * of the failing call), or "" if none.  Valid until the thread's next library call. */
const char* gemm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPGEMM_H */
