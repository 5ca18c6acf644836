// Device code of the software-pipelined tiled GEMM for gfx950 (MI355X).
//
//   C[M,N] = epi( A[M,K] . B ),  A row-major [M,K]; B row-major [K,N] ("kn") or [N,K] ("nk").
//
// The method is the output-stationary tiling with a pipelined K loop that the
// Mosaic GPU pipelining guide (Pallas) builds in "Example: matmul kernel on
// Hopper GPUs" and that the TileLang pipelined GEMM tutorial writes as
// T.Pipelined(ceildiv(K, block_K), num_stages): one workgroup owns a BM x BN
// block of C, holds its fp32 accumulator in registers across the whole K loop,
// and streams k-tiles of A and B through a ring of S shared-memory (LDS) slots
// so that the copies of later k-tiles overlap the matrix-core work on the
// current one.  What is specific to gfx950 here:
//
//  * Copies go straight from HBM/L2 to LDS with `buffer_load_dwordx4 ... lds`
//    (16 B per lane, 1 KiB per wave instruction), so no VGPRs stage the tiles.
//    A buffer resource per operand makes every access past the end of the
//    matrix return zero, which is how partial tiles read "other = 0"
//    (the masked loads of the Triton matmul in the Triton lecture notes).
//    Operands whose rows or base are not 16-byte aligned are staged through
//    VGPRs instead (copy mode 7, any 2-byte alignment).
//  * Each ring slot is its own __shared__ array and the K loop is unrolled over
//    the slot pattern, so every slot index is a compile-time constant.  The
//    compiler can then prove that the LDS reads of one slot do not alias the DMA
//    into another and does not insert a full `s_waitcnt vmcnt(0)` before them;
//    the kernel waits for exactly the copies it needs with `vmcnt(N)`.
//  * One barrier per k-tile, placed right after each wave's last LDS read of the
//    k-tile's slot, both publishes the next k-tile (every wave has waited for its
//    own copies of it) and releases the slot (MFMA reads registers, not LDS, so a
//    slot is free once every wave's reads of it have returned); the copies that
//    refill it are issued right after that barrier.  The guide's delay_release of
//    1 (refill one k-tile later) is copy mode 5.  B stored [K,N] on large grids
//    gets one more B slot than A slots (mode 6), so its copies have two k-tiles
//    to land.
//  * LDS tiles are XOR-swizzled at 16-byte granularity (the "swizzling" the
//    Triton notes give as the fix for bank conflicts, and the 128-byte swizzle
//    of the Pallas example) so that the 64 lanes of an operand read hit
//    distinct banks; the swizzle is applied by permuting the *global* chunk
//    each lane fetches, because direct-to-LDS writes land at lane*16.
//  * v_mfma_f32_16x16x32_{f16,bf16} on the 8-wave tiles the shape heuristic picks,
//    v_mfma_f32_32x32x16 on the misaligned-operand path and the 4-wave ablation tiles
//    (both shapes are compiled for the large tiles); the B tile is the first MFMA
//    operand and the A tile the second,
//    so each lane's accumulator holds consecutive output columns, which lets the
//    epilogue pack 4 outputs per LDS write.
//  * B stored [K,N] (N contiguous) is read with ds_read_b64_tr_b16, the
//    gfx950 transposing LDS read, instead of being transposed in registers.
//  * The instructions of a k-step are placed by hand, by the compiler, or (SCHED 2)
//    as a ping-pong of the two waves of each SIMD: one multiplies while the other
//    reads and copies, taking turns at a workgroup barrier.
//  * Epilogue: optional GELU or ReLU on the fp32 accumulator, round-to-nearest-even
//    conversion, staging through LDS (aliasing the drained ring), and 16-byte
//    row-contiguous global stores (the coalesced linear output traversal of
//    the XLA:GPU emitters page, loop emitter, with wider vectors), nontemporal
//    where C's rows are whole cache lines apart.
//  * Workgroup -> tile mapping gives each of the 8 XCDs a contiguous range of
//    tiles and rasterises tiles in groups of `group_m` tile rows, so the
//    workgroups that share an XCD's L2 share A and B panels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace spg {

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#define SPG_LDS __attribute__((address_space(3)))

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past any num_records: loads 0

enum { kOutF16 = 0, kOutBF16 = 1, kOutF32 = 2 };
enum { kEpiNone = 0, kEpiGelu = 1, kEpiRelu = 2 };

struct KArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;
    int32_t group_m;
    int32_t xcd_remap;
    int32_t out_dtype;
    int32_t epilogue;
    int32_t persistent;   // launcher only: run the persistent instantiation (grid = CUs)
    int32_t store_direct; // 1: the epilogue stores from registers, without LDS staging
    uint32_t* wait_timeouts;  // device word: bounded waits of the wave-specialized ring that gave up
    int32_t c_align;          // byte alignment of C's base address (1, 2, 4, 8 or 16)
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (V#) for a raw buffer of `bytes` bytes at `base`: any access at
// an offset >= bytes returns zero.  Word 3 = 0x00020000 selects the 32-bit data
// format of a raw (stride 0) buffer on gfx9.  The words are wave-uniform and
// are forced into SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)p);
    r.y = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(p >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r.w = 0x00020000;
    return r;
}

// One direct-to-LDS copy of 16 B per lane: the wave's 64 lanes land at LDS bytes
// [lds_dst, lds_dst + 1024), lane i at lds_dst + 16 i.  Written as inline asm on
// purpose: the compiler's wait-count pass cannot tell which LDS slot a DMA
// writes, and would otherwise wait for every outstanding copy before any LDS
// read, serializing the ring.  The kernel orders these copies itself with
// s_waitcnt vmcnt(N) and the per-k-tile barrier.  The asm writes M0 and lists it as
// clobbered; the compiler warns that M0 is a register it reserves.  These kernels
// (built for gfx950, where LDS instructions do not read M0 and every register array
// index is a compile-time constant) contain no M0 access of the compiler's own: in
// their assembly every M0 write is the one in this asm, one per LDS-DMA load.
__device__ __forceinline__ void dma16(const i32x4& rsrc, SPG_LDS char* lds_dst, uint32_t voff) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_dst);
    // s_nop: one wait state between the M0 write and the LDS-DMA load that reads it
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(m0), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// The 8 16-bit elements of a 16-byte chunk as one little-endian 128-bit number (element
// e in bits 16e .. 16e+15) shifted toward higher elements (shl) or lower ones (shr) by
// `bits` (a multiple of 16, 0 .. 112, per lane); zeros come in.  Realigns the chunks the
// misaligned-operand copy mode loads from a shifted window, and zeroes the elements of
// the window that lie outside the operand's valid range in the same step.
// Both are written as selects between values computed for either half, so that they
// compile to v_cndmask rather than to branches around per-lane conditions.
__device__ __forceinline__ u32x4 shl128(u32x4 v, uint32_t bits) {
    const uint64_t lo = ((uint64_t)v.y << 32) | v.x, hi = ((uint64_t)v.w << 32) | v.z;
    const uint32_t b = bits & 63u;              // shift within a 64-bit half
    // lo >> (64 - b) for b in 1 .. 63, written so that every shift count is < 64
    const uint64_t carry = b == 0 ? 0 : (lo >> 1) >> (63u - b);
    const bool big = bits >= 64;
    const uint64_t nhi = big ? lo << b : (hi << b) | carry;
    const uint64_t nlo = big ? 0 : lo << b;
    return u32x4{(uint32_t)nlo, (uint32_t)(nlo >> 32), (uint32_t)nhi, (uint32_t)(nhi >> 32)};
}

__device__ __forceinline__ u32x4 shr128(u32x4 v, uint32_t bits) {
    const uint64_t lo = ((uint64_t)v.y << 32) | v.x, hi = ((uint64_t)v.w << 32) | v.z;
    const uint32_t b = bits & 63u;
    const uint64_t carry = b == 0 ? 0 : (hi << 1) << (63u - b);
    const bool big = bits >= 64;
    const uint64_t nlo = big ? hi >> b : (lo >> b) | carry;
    const uint64_t nhi = big ? 0 : hi >> b;
    return u32x4{(uint32_t)nlo, (uint32_t)(nlo >> 32), (uint32_t)nhi, (uint32_t)(nhi >> 32)};
}

// Wait until at most N vector-memory instructions of this wave are outstanding.
// gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14];
// expcnt and lgkmcnt are left at their maxima (no wait on them).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Swizzle of K-contiguous tiles (A, and B stored [N,K]) with BK = 64: a row holds
// 64 halves = 8 chunks of 16 B; logical chunk c of row r lives at chunk c ^ kswz(r),
// kswz(r) = (r >> 1) & 7.  Rows 2j and 2j+1 (128 B apart) already fall on different
// banks, so only pairs of rows need distinct XOR values.  Chosen by measurement
// (SQ_LDS_BANK_CONFLICT over all 4096 XOR maps of the row's low 4 bits): 0% conflicts
// for both fragment reads, 32 rows x 2 chunks (32x32x16) and 16 rows x 4 chunks
// (16x16x32); the earlier (r & 7) ^ ((r >> 3) & 1) gave 0% and 25%.
// With BK = 32 a row is 4 chunks (64 B) and the XOR is ((r>>1) ^ (r>>2)) & 3:
// among 8 aligned rows, the 4 of equal parity (sharing a 128-B sweep) get
// distinct values, and among 16 aligned rows the 4 of equal r%4 (sharing a
// 256-B sweep) do too.
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }

// Swizzle of N-contiguous B tiles ([K,N] storage): the 16-B chunk index of row
// k is XOR-ed with {0, 6, 12, 10}[k & 3] ^ 2*(bit 3 of k).  A transposing read covers
// 4 consecutive rows; the table gives those 4 rows distinct 32-B windows within
// 128 B and distinct 64-B windows within 256 B, so one 16-lane group uses half of
// the banks.  The second term moves rows k+8 .. k+11 onto the other half: with
// 16x16x32 MFMAs the two 16-lane groups read together are rows k and k+8 of the
// same columns (with 32x32x16 they are the same rows, 16 columns apart, which the
// table alone separates).  Offsets of 4, 16 and 32 rows keep bit 3, so a lane's
// swizzle is fixed over the k-steps of a k-tile.
__device__ __forceinline__ int nswz(int k) { return ((0xAC60 >> ((k & 3) * 4)) & 15) ^ ((k >> 2) & 2); }

__device__ __forceinline__ float gelu_tanh(float x) {
    // 0.5 x (1 + tanh(u)) == x * sigmoid(2u) == x / (1 + exp(-2u)),
    // u = 0.7978845608 (x + 0.044715 x^3).  exp via v_exp_f32 (2^x); the
    // form saturates cleanly: exp -> inf gives -0, exp -> 0 gives x.
    // The one fused multiply-add is written out and contraction is off otherwise, so
    // every inlined copy (the staged and the direct epilogue, the standalone kernel)
    // rounds the same way and gives the same bits.
#pragma clang fp contract(off)
    const float x3 = 0.044715f * x * x;
    const float u = 0.7978845608f * __builtin_fmaf(x3, x, x);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);  // 2*log2(e) = 2.885...
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// max(x, 0) as the Triton lecture notes' matmul kernel applies it to the accumulator;
// a select (not fmaxf) so that -0 becomes +0 and the result is fully determined
__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

template <int EPI>
__device__ __forceinline__ float epi_t(float x) {
    if constexpr (EPI == kEpiGelu) return gelu_tanh(x);
    else if constexpr (EPI == kEpiRelu) return relu(x);
    else return x;
}

__device__ __forceinline__ float epi_apply(float x, int epi) {
    return epi == kEpiGelu ? gelu_tanh(x) : (epi == kEpiRelu ? relu(x) : x);
}

__device__ __forceinline__ uint16_t f32_to_bits(float x, bool bf16) {
    if (bf16) return __builtin_bit_cast(uint16_t, (__bf16)x);   // v_cvt_pk_bf16_f32, RNE
    // Without the empty asm the compiler may fold a preceding multiply into the
    // conversion (v_fma_mixlo_f16 a, b, 0): one rounding instead of two, and a -0
    // product comes out +0, so the bits would depend on the code around the call.
    asm("" : "+v"(x));
    return __builtin_bit_cast(uint16_t, (_Float16)x);            // v_cvt_f16_f32, RNE
}

__device__ __forceinline__ float bits_to_f32(uint16_t b, bool bf16) {
    if (bf16) return __builtin_bit_cast(float, (uint32_t)b << 16);
    return (float)__builtin_bit_cast(_Float16, b);
}

// Workgroup id -> (tile row, tile column).
__device__ __forceinline__ void tile_of(int wg, const KArgs& a, int& tm, int& tn) {
    const int T = a.tiles_m * a.tiles_n;
    if (a.xcd_remap) {
        // workgroups are dispatched round-robin over the 8 XCDs (wg % 8); hand XCD x
        // the contiguous tile range [x*q + min(x, r), ...) of its share
        const int x = wg & 7, i = wg >> 3, q = T >> 3, r = T & 7;
        wg = x * q + (x < r ? x : r) + i;
    }
    const int gsz = a.group_m * a.tiles_n;
    const int g = wg / gsz;
    const int first = g * a.group_m;
    const int rem = a.tiles_m - first;
    const int gm = rem < a.group_m ? rem : a.group_m;
    const int in = wg - g * gsz;
    tm = first + in % gm;
    tn = in / gm;
}

typedef float floatx4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_{f16,bf16}: x supplies rows 0..15 (lane l: row l%16, k 8(l/16)..+7),
// y columns 0..15 likewise; lane l receives D[4(l/16) + 0..3][l%16]
template <bool BF16>
__device__ __forceinline__ floatx4 mfma16(const u32x4& x, const u32x4& y, const floatx4& c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, x),
                                                      __builtin_bit_cast(halfx8, y), c, 0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ floatx16 mfma(const u32x4& x, const u32x4& y, const floatx16& c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                       __builtin_bit_cast(bf16x8, y), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, x),
                                                      __builtin_bit_cast(halfx8, y), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// the pipelined kernel
// ---------------------------------------------------------------------------

// Epilogue of one wave: accumulator -> (GELU / ReLU) -> output type -> LDS staging ->
// 16-byte row-contiguous global stores.  Where C's rows are whole 128-byte cache lines
// apart the stores are nontemporal: C is written once and never read here, and at the
// end of each round of tiles every workgroup stores its tile at once (32 MiB at 8192^3),
// which with the default policy evicts A/B panel lines the next round still needs
// (measured at 8192^3: NN -2.0%, TN -3.7% time).  Where they are not (N = 5000 with an
// fp32 C: rows 20,000 bytes apart), a tile's row segments share their first and last
// cache line with the neighbouring tiles; nontemporal writes of such partial lines are
// not merged, and there the default policy, which merges them in L2, is faster
// (3000x5000x1000 fp16 -> fp32: 45.4 -> 40.2 us; fp16 out 39.8 -> 36.3 us; 5000x3000 ->
// fp32 64.2 -> 59.7 us; shapes with line-multiple rows unchanged).  The wave's C tile is processed in 32-row
// blocks (one MFMA block row), NP blocks per round: a round writes its blocks into NP
// private 32 x WN staging buffers, then reads them back row by row and stores them, so
// the LDS write -> read -> store latency is paid once per round rather than per block.
// The 16-B chunks of a staged row are XOR-swizzled by row so that both the 4-value
// writes (32 rows, same column) and the row reads are free of bank conflicts.
template <int OD, int EPI, int TM, int TN, int WN, int NP = 1>
__device__ __forceinline__ void store_tile(const floatx16 (&acc)[TN][TM], char* stg,
                                           const KArgs& args, int m_base, int n_base, int lane) {
    constexpr int OB = OD == kOutF32 ? 4 : 2;         // output bytes
    constexpr int ROWB = WN * OB;                     // staged row bytes
    constexpr int CPR = ROWB / 16;                    // 16-B chunks per staged row
    constexpr int E16 = 16 / OB;                      // outputs per chunk
    constexpr int PASSB = 32 * ROWB;                  // staging bytes of one block
    static_assert(CPR == 8 || CPR == 16 || CPR == 32, "staging swizzle assumes 8..32 chunks");
    static_assert(NP >= 1 && TM % NP == 0, "blocks per round must divide the wave's blocks");
    auto swz = [](int row) { return CPR >= 16 ? (row & 15) : ((row >> 1) & 7); };
    const int M = args.M, N = args.N;
    // 16-byte stores need 16-byte rows and a 16-byte aligned C; otherwise element stores
    const bool vec_ok = (N % E16) == 0 && args.c_align >= 16;
    const bool nt_rows = ((size_t)N * OB) % 128 == 0;   // see the comment above
    const int lrow = lane & 31;
#pragma unroll
    for (int g = 0; g < TM; g += NP) {
        // one round at a time: keeps the accumulator reads of later rounds from being
        // hoisted into this one (with 256 accumulators that spills registers)
        __builtin_amdgcn_sched_barrier(0);
        // 1) lane holds C[row l%32][cols bn*32 + 8q + 4(l/32) + 0..3] of block g+p
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int bm = g + p;
            char* sp = stg + p * PASSB;
#pragma unroll
            for (int bn = 0; bn < TN; ++bn) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = acc[bn][bm][4 * q + e];
                        v[e] = epi_t<EPI>(v[e]);
                    }
                    const int byte = (bn * 32 + 8 * q + 4 * (lane >> 5)) * OB;
                    char* dst = sp + lrow * ROWB + (((byte >> 4) ^ swz(lrow)) << 4) + (byte & 15);
                    if constexpr (OD == kOutF32) {
                        *(SPG_LDS u32x4*)dst = u32x4{__builtin_bit_cast(uint32_t, v[0]),
                                                     __builtin_bit_cast(uint32_t, v[1]),
                                                     __builtin_bit_cast(uint32_t, v[2]),
                                                     __builtin_bit_cast(uint32_t, v[3])};
                    } else {
                        constexpr bool BF = OD == kOutBF16;
                        const uint32_t p0 = (uint32_t)f32_to_bits(v[0], BF) | ((uint32_t)f32_to_bits(v[1], BF) << 16);
                        const uint32_t p1 = (uint32_t)f32_to_bits(v[2], BF) | ((uint32_t)f32_to_bits(v[3], BF) << 16);
                        *(SPG_LDS u32x2*)dst = u32x2{p0, p1};
                    }
                }
            }
        }
        // 2) LDS -> global, 16 B per lane, consecutive lanes along a row
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int bm = g + p;
            const char* sp = stg + p * PASSB;
#pragma unroll 1
            for (int it = 0; it < (32 * CPR) / 64; ++it) {
                const int idx = it * 64 + lane;
                const int row = idx / CPR;
                const int ch = idx % CPR;
                const u32x4 val = *(const SPG_LDS u32x4*)(sp + row * ROWB + ((ch ^ swz(row)) << 4));
                const int gm = m_base + bm * 32 + row;
                const int gn = n_base + ch * E16;
                if (gm < M && gn < N) {
                    char* dstg = (char*)args.C + ((size_t)gm * N + gn) * OB;
                    if (vec_ok && gn + E16 <= N) {
                        if (nt_rows) __builtin_nontemporal_store(val, (u32x4*)dstg);
                        else *(u32x4*)dstg = val;
                    } else {
                        const int lim = (N - gn) < E16 ? (N - gn) : E16;
                        for (int e = 0; e < lim; ++e) {
                            if constexpr (OB == 4) ((uint32_t*)dstg)[e] = val[e];
                            else ((uint16_t*)dstg)[e] = (uint16_t)(val[e >> 1] >> ((e & 1) * 16));
                        }
                    }
                }
            }
        }
    }
}

// The staged epilogue for 16x16x32 accumulators: lane l holds C[bm*16 + l%16][bn*16 +
// 4(l/16) + 0..3]; a staged 32-row block is the accumulators of bm = 2g and 2g+1.  The
// staging layout and the read-back are those of store_tile.
template <int OD, int EPI, int TM, int TN, int WN, int NP = 1>
__device__ __forceinline__ void store_tile16(const floatx4 (&acc)[TN][TM], char* stg,
                                             const KArgs& args, int m_base, int n_base, int lane) {
    constexpr int OB = OD == kOutF32 ? 4 : 2;
    constexpr int ROWB = WN * OB;
    constexpr int CPR = ROWB / 16;
    constexpr int E16 = 16 / OB;
    constexpr int PASSB = 32 * ROWB;
    constexpr int NB32 = TM / 2;                      // 32-row blocks
    static_assert(CPR == 8 || CPR == 16 || CPR == 32, "staging swizzle assumes 8..32 chunks");
    static_assert(TM % 2 == 0 && NB32 % NP == 0, "blocks per round must divide the wave's blocks");
    auto swz = [](int row) { return CPR >= 16 ? (row & 15) : ((row >> 1) & 7); };
    const int M = args.M, N = args.N;
    const bool vec_ok = (N % E16) == 0 && args.c_align >= 16;
    const bool nt_rows = ((size_t)N * OB) % 128 == 0;   // the store policy of store_tile
    const int lrow = lane & 15;
#pragma unroll
    for (int g = 0; g < NB32; g += NP) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            char* sp = stg + p * PASSB;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int bm = 2 * (g + p) + h;
                const int row = h * 16 + lrow;
#pragma unroll
                for (int bn = 0; bn < TN; ++bn) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = epi_t<EPI>(acc[bn][bm][e]);
                    const int byte = (bn * 16 + 4 * (lane >> 4)) * OB;
                    char* dst = sp + row * ROWB + (((byte >> 4) ^ swz(row)) << 4) + (byte & 15);
                    if constexpr (OD == kOutF32) {
                        *(SPG_LDS u32x4*)dst = u32x4{__builtin_bit_cast(uint32_t, v[0]),
                                                     __builtin_bit_cast(uint32_t, v[1]),
                                                     __builtin_bit_cast(uint32_t, v[2]),
                                                     __builtin_bit_cast(uint32_t, v[3])};
                    } else {
                        constexpr bool BF = OD == kOutBF16;
                        const uint32_t p0 = (uint32_t)f32_to_bits(v[0], BF) | ((uint32_t)f32_to_bits(v[1], BF) << 16);
                        const uint32_t p1 = (uint32_t)f32_to_bits(v[2], BF) | ((uint32_t)f32_to_bits(v[3], BF) << 16);
                        *(SPG_LDS u32x2*)dst = u32x2{p0, p1};
                    }
                }
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const char* sp = stg + p * PASSB;
#pragma unroll 1
            for (int it = 0; it < (32 * CPR) / 64; ++it) {
                const int idx = it * 64 + lane;
                const int row = idx / CPR;
                const int ch = idx % CPR;
                const u32x4 val = *(const SPG_LDS u32x4*)(sp + row * ROWB + ((ch ^ swz(row)) << 4));
                const int gm = m_base + (g + p) * 32 + row;
                const int gn = n_base + ch * E16;
                if (gm < M && gn < N) {
                    char* dstg = (char*)args.C + ((size_t)gm * N + gn) * OB;
                    if (vec_ok && gn + E16 <= N) {
                        if (nt_rows) __builtin_nontemporal_store(val, (u32x4*)dstg);
                        else *(u32x4*)dstg = val;
                    } else {
                        const int lim = (N - gn) < E16 ? (N - gn) : E16;
                        for (int e = 0; e < lim; ++e) {
                            if constexpr (OB == 4) ((uint32_t*)dstg)[e] = val[e];
                            else ((uint16_t*)dstg)[e] = (uint16_t)(val[e >> 1] >> ((e & 1) * 16));
                        }
                    }
                }
            }
        }
    }
}

// Epilogue without LDS staging (the ablation of the staged one), 16-bit outputs: each
// lane stores its own accumulator values, 4 consecutive outputs of one row per store,
// so one wave instruction writes 32 rows x 2 segments of 8 bytes.  The epilogue and the
// output type are applied per value at run time: one instantiation per kernel.
template <int TM, int TN, int MI, typename AccV>
__device__ __forceinline__ void store_direct16(const AccV (&acc)[TN][TM], const KArgs& args,
                                               int m_base, int n_base, int lane) {
    constexpr int QN = MI == 32 ? 4 : 1;   // 4-output segments per accumulator tile and lane
    const int M = args.M, N = args.N;
    const int ep = args.epilogue;
    const bool bf = args.out_dtype == kOutBF16;
    const bool vec_ok = (N % 4) == 0 && args.c_align >= 8;    // every 4-output segment 8-byte aligned
#pragma unroll
    for (int bm = 0; bm < TM; ++bm) {
        __builtin_amdgcn_sched_barrier(0);
        const int gm = m_base + bm * MI + (lane & (MI - 1));
#pragma unroll
        for (int bn = 0; bn < TN; ++bn) {
#pragma unroll
            for (int q = 0; q < QN; ++q) {
                uint32_t h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = epi_apply(acc[bn][bm][4 * q + e], ep);
                    h[e] = bf ? (uint32_t)f32_to_bits(x, true) : (uint32_t)f32_to_bits(x, false);
                }
                const int gn = MI == 32 ? n_base + bn * 32 + 8 * q + 4 * (lane >> 5)
                                        : n_base + bn * 16 + 4 * (lane >> 4);
                if (gm < M && gn < N) {
                    uint16_t* dst = (uint16_t*)args.C + ((size_t)gm * N + gn);
                    if (vec_ok && gn + 4 <= N) {
                        __builtin_nontemporal_store(u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)}, (u32x2*)dst);
                    } else {
                        const int lim = (N - gn) < 4 ? (N - gn) : 4;
                        for (int e = 0; e < lim; ++e) dst[e] = (uint16_t)h[e];
                    }
                }
            }
        }
    }
}

// Largest number of 32-row blocks (a divisor of TM) whose staging fits `budget` bytes.
template <int TM, int WN, int OB>
constexpr int blocks_per_round(int budget) {
    int np = 1;
    for (int d = 1; d <= TM; ++d)
        if (TM % d == 0 && d * 32 * WN * OB <= budget) np = d;
    return np;
}

// Poisoned ring (a test instrument, compiled only into the separate poison library with
// -DSPG_POISON): the ring starts as NaN, and the moment the barrier protocol releases a
// region of a slot, the wave that will refill it first overwrites it with NaN (all-ones
// halves: NaN in both fp16 and bf16).  A fragment read that the protocol does not cover,
// of a k-tile whose copies have not landed and been published, or of a slot already
// released, then reads NaN rather than a plausible stale or early k-tile, the NaN reaches
// every output of the MFMA tile, and a parity test cannot miss it.  The write-after-read
// window widens from "until the refill lands" (hundreds of cycles) to "from the release
// barrier on".
#ifdef SPG_POISON
constexpr bool kPoison = true;
#else
constexpr bool kPoison = false;
#endif

// Workgroup barrier for LDS hazards only: this wave's LDS operations have
// completed (lgkmcnt(0)) and every wave has arrived.  Unlike __syncthreads it
// does not wait for outstanding global loads, so staged loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_b(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

template <int BM, int BN, int BK, int WM, int WN, int S, int MI = 32>
struct Geom {
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NW = (BM / WM) * WAVES_N;
    static constexpr int NT = NW * 64;
    // MFMA tiles per wave: MI x MI outputs each (32x32x16 or 16x16x32)
    static constexpr int TM = WM / MI, TN = WN / MI;
    static constexpr int KPS = MI == 32 ? 16 : 32;     // k of one MFMA step
    static constexpr int KSTEPS = BK / KPS;            // MFMA k-steps per k-tile
    static_assert(MI == 32 || MI == 16, "MFMA shape");
    static constexpr int ROWB = BK * 2;                // bytes of a K-contiguous tile row
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BN * BK * 2;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_DMA = A_BYTES / 1024 / NW;  // DMA instructions per wave per k-tile
    static constexpr int B_DMA = B_BYTES / 1024 / NW;
    static constexpr int L = A_DMA + B_DMA;
    static constexpr int STG = 32 * WN * 4;            // epilogue staging bytes of one fp32 block
    // epilogue staging available per wave: a ring slot shared by ceil(NW / S) waves
    static constexpr int STGW = (STAGE / ((NW + S - 1) / S)) / 16 * 16;
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(BM % WM == 0 && BN % WN == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(BN >= 128, "[K,N] swizzle needs 16 chunks per row");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "DMA split");
    static_assert(S >= 1 && S <= 6, "stages");
    static_assert(S * STAGE <= 160 * 1024, "LDS budget");
    static_assert(((NW + S - 1) / S) * STG <= STAGE, "epilogue staging must fit the ring");
    static_assert((S > 2 ? (S - 2) * L : 0) < 64, "vmcnt range");
};

// Swizzle of a K-contiguous tile row with BK/8 chunks of 16 B (both maps are described at kswz).
template <int BK>
__device__ __forceinline__ int kswz_t(int r) {
    if constexpr (BK == 64) return kswz(r);
    else return ((r >> 1) ^ (r >> 2)) & 3;
}

// LDM selects how a k-tile reaches its LDS slot:
//   0  direct-to-LDS copies (buffer_load ... lds), no VGPR staging, all copies of
//      k-tile t+S issued in the stage right after the barrier that frees slot t;
//   1  register-staged: buffer_load_dwordx4 into VGPRs one k-tile ahead, then
//      ds_write_b128 into the same swizzled slot layout.  LDS writes from VGPRs
//      leave the LDS more read bandwidth than direct copies do.
//   2  direct-to-LDS copies spread evenly over the whole window from one barrier
//      to the next (L / KSTEPS per stage), so the vector-memory queue never
//      backs up into the MFMA issue of a wave that is alone on its SIMD.  The
//      last copies of a window land one k-tile before they are read, hence S >= 3.
//   4  direct-to-LDS copies as in 0, with the A operand in a ring one slot deeper
//      than B (S = 2: three A slots, two B slots).  The window after barrier t copies
//      B of k-tile t+2 and A of k-tile t+3, so A has two k-tiles to land instead of
//      one; the B copies are issued first, and the wait before barrier t+1 leaves the
//      A copies of k-tile t+3 in flight.  With the tile raster's 8 x 4 blocks of
//      tiles per XCD, A carries 2/3 of the bytes that miss L2.  The loop is unrolled
//      by 6 k-tiles (three A slots x two B slots), plus an unrolled tail.
//   6  the mirror of 4: B in a ring one slot deeper than A (two A slots, three B
//      slots).  The window after barrier t copies A of k-tile t+2, then B of k-tile
//      t+3, and the wait before barrier t+1 leaves the B copies in flight.  With the
//      16x16x32 tiles it fits the registers only under the compiler's schedule
//      (SCHED 1; the hand-placed one spills), and there it is the fastest measured
//      configuration at bf16 8192^3 (NN -1.3% time against mode 0 hand-placed).
//   7  register-staged as in 1, for operands whose rows or base addresses are not 16-byte
//      aligned (K % 8 != 0, B stored [K,N] with N % 8 != 0, or a base pointer that is
//      not 16-byte aligned): each lane loads its 16 bytes with a buffer_load_dwordx4 at
//      any 2-byte alignment (ROCm runs compute queues in unaligned-access mode, which the
//      gfx950 code generation assumes as well).  The partial k-tile may then start at any
//      element: on k-tile 0 a chunk that straddles k = 0 is loaded from the window that
//      starts at k = 0 and shifted up by the straddle (shl128), which also zeroes its k < 0
//      elements.  For B stored [K,N], a chunk that straddles column N is loaded from the
//      window that ends at column N (never past the end of B) and shifted down (shr128),
//      zeroing its columns >= N.  Rows past M (A) or N (B stored [N,K]) read zero through
//      the buffer resource as in the other modes.
//   5  direct-to-LDS copies as in 0, but a slot is refilled one k-tile after its
//      release (the release delay of 1 in the Pallas guide's terms): the window
//      after barrier t copies k-tile t+S-1 into the slot released at barrier t-1, so
//      S-1 k-tiles are in flight instead of S (needs S >= 3).  Mode 0 refills a slot
//      at the barrier that releases it, which is the same barrier that publishes the
//      next k-tile: no second barrier is needed for the early release.
//
// PF (lookahead) is the number of MFMA k-steps between the LDS read of an operand
// fragment and its use: 1 keeps two fragment sets in registers, 2 keeps four and
// gives every read a whole extra stage to return, which a wave alone on its SIMD
// needs when the LDS is busy.  The barrier of a k-tile sits PF stages before its
// end, right after the last read of the slot.
//
// SCHED selects who places the instructions of a stage: 0 = by hand, every MFMA
// step followed by its copy op and LDS reads and a scheduling barrier (the
// TileLang tutorial's manual stage/order placement); 1 = the compiler, with the
// same instructions and no scheduling barriers (its compiler-planned pipeline);
// 2 = ping-pong: the two waves of a SIMD take turns, one issuing only MFMAs while
// the other reads fragments and copies, with a workgroup barrier between turns
// (B-deep ring, 16x16x32, 8 waves; the K loop's comment has the protocol).
//
// PERS (persistent): the grid holds one workgroup per CU and workgroup w computes
// tiles w, w + G, w + 2G, ... (G = grid size) as one continuous stream of k-tiles,
// so the copies issued during the last k-tiles of a tile already fetch the first
// k-tiles of the next one, and the fragment lookahead runs across the tile
// boundary.  Each tile's epilogue goes through a staging area of its own (the ring
// stays busy with the next tile's copies) and no workgroup-wide barrier is added.
// The launcher uses it only when K % BK == 0 (no partial k-tile), the output is
// 16-bit and, for B stored [K,N], N % BN == 0 (no column masks on the copies).
//
// MI selects the MFMA: 32 = v_mfma_f32_32x32x16 (16 accumulators per lane and tile, k 16
// per step), 16 = v_mfma_f32_16x16x32 (4 accumulators per lane and tile, k 32 per step).
// The LDS layout, the copies and the ring are the same; the fragment reads, the MFMA
// call and the epilogue's accumulator layout differ.
template <bool BF16, bool B_NK, int BM, int BN, int BK, int WM, int WN, int S, bool SWZ, int LDM,
          int PF, int SCHED, bool PERS, int MI>
__global__ void __launch_bounds__((Geom<BM, BN, BK, WM, WN, S, MI>::NT))
pipelined_gemm(KArgs args) {
    using G = Geom<BM, BN, BK, WM, WN, S, MI>;
    static_assert(MI == 32 || (!PERS && PF == 1 && BK == 64), "16x16x32: BK 64, lookahead 1, one workgroup per tile");
    static_assert(LDM != 2 || S >= 3, "spread copies need a slot of slack");
    static_assert(PF == 1 || (PF == 2 && BK == 64 && S > 1), "lookahead 2 needs four k-steps per k-tile");
    static_assert(!PERS || (LDM == 0 && S >= 2), "persistent: direct copies and a ring of >= 2 slots");
    static_assert(LDM != 4 || (S == 2 && S * G::STAGE + G::A_BYTES <= 160 * 1024),
                  "A-deep ring: two slots plus one more A slot within the LDS");
    static_assert(LDM != 6 || (S == 2 && S * G::STAGE + G::B_BYTES <= 160 * 1024),
                  "B-deep ring: two slots plus one more B slot within the LDS");
    static_assert(LDM != 5 || S >= 3, "a late release needs a ring of three slots or more");
    static_assert(LDM != 7 || (S >= 2 && !PERS), "misaligned operands: register staging, ring of >= 2 slots");
    static_assert(!PERS || S * G::STAGE + G::NW * 32 * WN * 2 <= 160 * 1024,
                  "persistent: ring + epilogue staging must fit the LDS");
    constexpr int TM = G::TM, TN = G::TN, A_BYTES = G::A_BYTES, KSTEPS = G::KSTEPS;
    constexpr int ROWB = G::ROWB;
    constexpr int A_DMA = G::A_DMA, B_DMA = G::B_DMA;
    constexpr int CPR_K = BK / 8;          // chunks per K-contiguous row
    constexpr int RPI_K = 64 / CPR_K;      // K-contiguous rows per DMA instruction

    __shared__ __attribute__((aligned(1024))) char ring0[G::STAGE];
    __shared__ __attribute__((aligned(1024))) char ring1[S > 1 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char ring2[S > 2 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char ring3[S > 3 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char ring4[S > 4 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char ring5[S > 5 ? G::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char ring_a2[LDM == 4 ? G::A_BYTES : 16];
    __shared__ __attribute__((aligned(1024))) char ring_b2[LDM == 6 ? G::B_BYTES : 16];

    // ring slot s as a compile-time choice of array (see the header comment); a slot
    // is addressed through its A and B parts, which the A-deep and B-deep rings (LDM 4
    // and 6) place in different arrays
    struct Slot {
        SPG_LDS char* a;
        SPG_LDS char* b;
    };
    auto ring_of = [&](auto sc) -> SPG_LDS char* {
        constexpr int v = decltype(sc)::value;
        if constexpr (v == 0) return (SPG_LDS char*)ring0;
        else if constexpr (v == 1) return (SPG_LDS char*)ring1;
        else if constexpr (v == 2) return (SPG_LDS char*)ring2;
        else if constexpr (v == 3) return (SPG_LDS char*)ring3;
        else if constexpr (v == 4) return (SPG_LDS char*)ring4;
        else return (SPG_LDS char*)ring5;
    };
    auto slot_of = [&](auto sc) -> Slot {
        SPG_LDS char* r = ring_of(sc);
        return Slot{r, r + G::A_BYTES};
    };
    // slot of k-tile t for t % 6 == i in the A-deep ring: A in the A part of ring0,
    // ring1 or in ring_a2 (t % 3), B in the B part of ring0 or ring1 (t % 2).  The
    // B-deep ring (LDM 6) mirrors it: A in ring0/ring1 (t % 2), B in the B part of
    // ring0, ring1 or in ring_b2 (t % 3)
    auto deep_slot = [&](auto ic) -> Slot {
        constexpr int i = decltype(ic)::value;
        if constexpr (LDM == 6) {
            SPG_LDS char* a = (i % 2) == 0 ? (SPG_LDS char*)ring0 : (SPG_LDS char*)ring1;
            SPG_LDS char* b = (i % 3) == 0 ? (SPG_LDS char*)ring0 + G::A_BYTES
                            : (i % 3) == 1 ? (SPG_LDS char*)ring1 + G::A_BYTES : (SPG_LDS char*)ring_b2;
            return Slot{a, b};
        }
        SPG_LDS char* a = (i % 3) == 0 ? (SPG_LDS char*)ring0
                        : (i % 3) == 1 ? (SPG_LDS char*)ring1 : (SPG_LDS char*)ring_a2;
        SPG_LDS char* b = ((i % 2) == 0 ? (SPG_LDS char*)ring0 : (SPG_LDS char*)ring1) + G::A_BYTES;
        return Slot{a, b};
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // the wave index is uniform: kept in an SGPR, so are the copy addresses derived from it
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / G::WAVES_N;
    const int wn = wave % G::WAVES_N;

    constexpr u32x4 kNaN16 = {~0u, ~0u, ~0u, ~0u};
    if constexpr (kPoison) {
        // the poison build: every slot starts as NaN
        auto fill = [&](char* p, int bytes) {
            for (int o = tid * 16; o < bytes; o += G::NT * 16) *(u32x4*)(p + o) = kNaN16;
        };
        // (only the arrays this configuration uses: touching a placeholder would allocate it)
        fill(ring0, sizeof ring0);
        if constexpr (S > 1) fill(ring1, sizeof ring1);
        if constexpr (S > 2) fill(ring2, sizeof ring2);
        if constexpr (S > 3) fill(ring3, sizeof ring3);
        if constexpr (S > 4) fill(ring4, sizeof ring4);
        if constexpr (S > 5) fill(ring5, sizeof ring5);
        if constexpr (LDM == 4) fill(ring_a2, sizeof ring_a2);
        if constexpr (LDM == 6) fill(ring_b2, sizeof ring_b2);
        __syncthreads();
    }

    int tm, tn;
    tile_of(blockIdx.x, args, tm, tn);
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (K + BK - 1) / BK;
    // k-tile kt covers k in [kt*BK - pad, kt*BK - pad + BK) with pad = (-K) mod BK:
    // the partial k-tile, when K % BK != 0, is the first one and its k < 0 part
    // reads as zeros.  Every later k-tile lies inside [0, K), so only the copies
    // of k-tile 0 (all issued before the K loop) carry per-lane masks.  pad is a
    // multiple of 8 (K % 8 == 0), i.e. of the 16-byte copy granule, except in copy
    // mode 7, where the chunk that straddles k = 0 is realigned (see the mode list).
    const int pad = (BK - K % BK) % BK;
    constexpr bool UNAL = LDM == 7;                 // misaligned-operand copy mode
    constexpr bool REG = LDM == 1 || LDM == 7;      // k-tiles staged through VGPRs

    // ---- copy sources: one buffer resource per operand and k-tile -------------
    // The resource of k-tile kt starts at the tile's first k and ends where this
    // workgroup's rows of the operand end, so rows past M (A) or past N (B stored
    // [N,K]) read as zero; past the last k-tile it is empty and reads zero.  The
    // per-lane offsets inside it are the same for every k-tile, so a copy is one
    // M0 write and one buffer_load; the per-k-tile work is scalar.
    const int a_rows = (M - m0) < BM ? (M - m0) : BM;
    const uint64_t a_base = (uint64_t)(uintptr_t)(args.A + (size_t)m0 * K);
    const uint32_t a_bytes = (uint32_t)a_rows * (uint32_t)K * 2u;
    uint64_t b_base;
    uint32_t b_bytes, b_kb;  // b_kb: bytes between consecutive k
    if constexpr (B_NK) {
        const int b_rows = (N - n0) < BN ? (N - n0) : BN;
        b_base = (uint64_t)(uintptr_t)(args.B + (size_t)n0 * K);
        b_bytes = (uint32_t)b_rows * (uint32_t)K * 2u;
        b_kb = 2u;
    } else {
        b_base = (uint64_t)(uintptr_t)(args.B + n0);
        b_bytes = (uint32_t)(((size_t)K * N - n0) * 2u);
        b_kb = 2u * (uint32_t)N;
        if constexpr (UNAL) {
            // in mode 7 the window of a chunk that straddles N starts up to 7 columns
            // before n0 when the last column tile holds fewer than 8 columns: the resource
            // starts 16 bytes earlier so that every window offset is non-negative (an
            // offset is an unsigned 32-bit value; a negative one would read zero)
            b_base -= 16u;
            b_bytes += 16u;
        }
    }
    // start address and size of an operand's resource for k-tile kt
    auto window = [&](uint64_t base, uint32_t bytes, uint32_t kb, int kt, uint64_t& p,
                      uint32_t& nr) __attribute__((always_inline)) {
        const int64_t shift = (int64_t)(kt * BK - pad) * (int64_t)kb;  // < 0 only for kt = 0
        p = base + (uint64_t)shift;
        nr = kt < nk ? bytes - (uint32_t)shift : 0u;
    };
    struct DmaSrc { i32x4 a, b; };
    auto dma_src = [&](int kt) __attribute__((always_inline)) -> DmaSrc {
        uint64_t pa, pb;
        uint32_t na, nb;
        window(a_base, a_bytes, 2u, kt, pa, na);
        window(b_base, b_bytes, b_kb, kt, pb, nb);
        return DmaSrc{make_rsrc((const void*)(uintptr_t)pa, na), make_rsrc((const void*)(uintptr_t)pb, nb)};
    };
    struct RegSrc { __amdgpu_buffer_rsrc_t a, b; };
    auto reg_src = [&](int kt) __attribute__((always_inline)) -> RegSrc {
        uint64_t pa, pb;
        uint32_t na, nb;
        window(a_base, a_bytes, 2u, kt, pa, na);
        window(b_base, b_bytes, b_kb, kt, pb, nb);
        return RegSrc{make_rsrc_b((const void*)(uintptr_t)pa, na), make_rsrc_b((const void*)(uintptr_t)pb, nb)};
    };

    // ---- per-lane copy offsets -----------------------------------------------
    // Copy instruction d of a k-tile writes LDS bytes [d*1024, d*1024+1024): lane i
    // lands at byte i*16, i.e. row d*RPI + i/CPR, physical chunk i%CPR; it fetches
    // the logical chunk that the swizzle puts there.  kinA/kinB: the k offset of the
    // lane's 8 elements inside the k-tile, for the masks of k-tile 0.  Columns past
    // N of a [K,N] B point past every resource and read as zero; in mode 7 a chunk that
    // straddles N is loaded from the window ending at N and shifted down by the number
    // of its columns past N, kept in 3 bits per op of nsh_pack (one register).
    uint32_t offA[A_DMA];
    int kinA[A_DMA];
#pragma unroll
    for (int j = 0; j < A_DMA; ++j) {
        const int d = wave * A_DMA + j;
        const int r = d * RPI_K + lane / CPR_K;
        const int p = lane % CPR_K;
        const int c = SWZ ? (p ^ kswz_t<BK>(r)) : p;
        offA[j] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)c * 16u;
        kinA[j] = c * 8;
    }
    uint32_t offB[B_DMA];
    int kinB[B_DMA];
    uint32_t nsh_pack = 0;
    static_assert(3 * B_DMA <= 32, "column shifts packed 3 bits per op");
#pragma unroll
    for (int j = 0; j < B_DMA; ++j) {
        const int d = wave * B_DMA + j;
        if constexpr (B_NK) {
            const int r = d * RPI_K + lane / CPR_K;
            const int p = lane % CPR_K;
            const int c = SWZ ? (p ^ kswz_t<BK>(r)) : p;
            offB[j] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)c * 16u;
            kinB[j] = c * 8;
        } else {
            constexpr int CPR = BN / 8;          // 16-B chunks per [K,N] row
            constexpr int RP = 64 / CPR;         // rows per wave instruction
            const int r = d * RP + lane / CPR;
            const int p = lane % CPR;
            const int c = SWZ ? (p ^ nswz(r)) : p;
            const int over = n0 + c * 8 + 8 - N;    // columns of the chunk at or past N
            if constexpr (UNAL) {
                offB[j] = over >= 8 ? kOOB
                                    : 16u + (uint32_t)r * (uint32_t)N * 2u + (uint32_t)c * 16u
                                          - (over > 0 ? 2u * (uint32_t)over : 0u);
                nsh_pack |= (over > 0 && over < 8 ? (uint32_t)over : 0u) << (3 * j);
            } else {
                offB[j] = over > 0 ? kOOB : (uint32_t)r * (uint32_t)N * 2u + (uint32_t)c * 16u;
            }
            kinB[j] = r;
        }
    }

    // Offset of copy op j (compile-time): j < A_DMA moves A rows, the rest B.  On
    // k-tile 0 (FIRST) the lanes whose elements lie at k < 0 read zero; in mode 7 a
    // K-contiguous chunk with only some elements at k < 0 reads the window that starts
    // at k = 0 (kin + 8 > pad > kin), realigned by k0_shift before its LDS write.
    auto first_off = [&](uint32_t off, int kin, bool k_contiguous) __attribute__((always_inline)) -> uint32_t {
        if (kin >= pad) return off;
        if (!UNAL || !k_contiguous || kin + 8 <= pad) return kOOB;
        return off + 2u * (uint32_t)(pad - kin);
    };
    auto src_off = [&](auto jc, auto first) __attribute__((always_inline)) -> uint32_t {
        constexpr int j = decltype(jc)::value;
        constexpr bool FIRST = decltype(first)::value;
        if constexpr (j < A_DMA) {
            if constexpr (FIRST) return first_off(offA[j], kinA[j], true);
            else return offA[j];
        } else {
            constexpr int jb = j - A_DMA;
            if constexpr (FIRST) return first_off(offB[jb], kinB[jb], B_NK);
            else return offB[jb];
        }
    };
    // mode 7, k-tile 0: bits to shift a K-contiguous chunk that straddles k = 0 up by
    auto k0_shift = [&](int kin) __attribute__((always_inline)) -> uint32_t {
        return kin < pad && kin + 8 > pad ? 16u * (uint32_t)(pad - kin) : 0u;
    };
    // op j writes LDS bytes lds_off(j) + 16*lane of the slot's A part (j < A_DMA) or
    // B part
    auto lds_off = [&](auto jc) __attribute__((always_inline)) -> int {
        constexpr int j = decltype(jc)::value;
        if constexpr (j < A_DMA) return (wave * A_DMA + j) * 1024;
        else return (wave * B_DMA + (j - A_DMA)) * 1024;
    };
    auto part = [&](const Slot& slot, auto jc) __attribute__((always_inline)) -> SPG_LDS char* {
        return decltype(jc)::value < A_DMA ? slot.a : slot.b;
    };
    using NotFirst = std::false_type;
    using First = std::true_type;
    auto dma_op = [&](const Slot& slot, const DmaSrc& src, auto jc, auto first)
                      __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        dma16(j < A_DMA ? src.a : src.b, part(slot, jc) + lds_off(jc), src_off(jc, first));
    };
    // register staging (LDM 1 and 7): one k-tile of copies in flight in VGPRs
    u32x4 stage_regs[G::L];
    auto gload_op = [&](const RegSrc& src, auto jc, auto first) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        stage_regs[j] = __builtin_amdgcn_raw_buffer_load_b128(j < A_DMA ? src.a : src.b,
                                                              (int)src_off(jc, first), 0, 0);
    };
    // write op j of the staged k-tile (FIRST: k-tile 0) into its slot; mode 7 realigns it
    auto lwrite_op = [&](const Slot& slot, auto jc, auto first) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        constexpr bool FIRST = decltype(first)::value;
        u32x4 v = stage_regs[j];
        if constexpr (UNAL) {
            if constexpr (j < A_DMA) {
                if constexpr (FIRST) v = shl128(v, k0_shift(kinA[j]));
            } else if constexpr (B_NK) {
                if constexpr (FIRST) v = shl128(v, k0_shift(kinB[j - A_DMA]));
            } else {
                v = shr128(v, 16u * ((nsh_pack >> (3 * (j - A_DMA))) & 7u));
            }
        }
        *(SPG_LDS u32x4*)(part(slot, jc) + lds_off(jc) + lane * 16) = v;
    };
    auto issue = [&](const Slot& slot, int kt, auto first) __attribute__((always_inline)) {
        const DmaSrc src = dma_src(kt);
        static_for<0, G::L>([&](auto jc) { dma_op(slot, src, jc, first); });
    };
    // the poison build: NaN over every region of `slot` that this wave's copy ops write.
    // Direct-to-LDS copies write the LDS outside the wave's LDS queue, so the NaN must
    // have landed (lgkmcnt(0)) before they are issued; a register-staged refill is an
    // LDS write of the same wave, which the LDS executes in order after the NaN.
    auto poison_slot = [&](const Slot& slot) __attribute__((always_inline)) {
        if constexpr (kPoison) {
            static_for<0, G::L>([&](auto jc) {
                *(SPG_LDS u32x4*)(part(slot, jc) + lds_off(jc) + lane * 16) = kNaN16;
            });
            if constexpr (!REG) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    };

    // ---- persistent: the copy side of the k-tile stream ------------------------
    // (cp_tile, cp_kt) is the next k-tile to copy; cp_* hold the resource bases of
    // cp_tile (empty once it is past the last tile: those copies read zero).
    const int T = args.tiles_m * args.tiles_n;
    int cp_tile = blockIdx.x, cp_kt = 0;
    bool cp_valid = false;
    uint64_t cp_a = 0, cp_b = 0;
    uint32_t cp_an = 0, cp_bn = 0;
    auto set_copy_tile = [&]() __attribute__((always_inline)) {
        cp_valid = cp_tile < T;
        if (cp_valid) {
            int ctm, ctn;
            tile_of(cp_tile, args, ctm, ctn);
            const int cm0 = ctm * BM, cn0 = ctn * BN;
            const int ar = (M - cm0) < BM ? (M - cm0) : BM;
            cp_a = (uint64_t)(uintptr_t)(args.A + (size_t)cm0 * K);
            cp_an = (uint32_t)ar * (uint32_t)K * 2u;
            if constexpr (B_NK) {
                const int br = (N - cn0) < BN ? (N - cn0) : BN;
                cp_b = (uint64_t)(uintptr_t)(args.B + (size_t)cn0 * K);
                cp_bn = (uint32_t)br * (uint32_t)K * 2u;
            } else {
                cp_b = (uint64_t)(uintptr_t)(args.B + cn0);
                cp_bn = (uint32_t)(((size_t)K * N - cn0) * 2u);
            }
        }
    };
    // resources of the next k-tile of the stream, then advance (K % BK == 0: every
    // k-tile of a valid tile lies inside [0, K), so the window never underflows)
    auto next_copy = [&]() __attribute__((always_inline)) -> DmaSrc {
        const uint32_t sa = (uint32_t)cp_kt * (uint32_t)(BK * 2);
        const uint32_t sb = (uint32_t)cp_kt * (uint32_t)BK * b_kb;
        const DmaSrc r{make_rsrc((const void*)(uintptr_t)(cp_a + sa), cp_valid ? cp_an - sa : 0u),
                       make_rsrc((const void*)(uintptr_t)(cp_b + sb), cp_valid ? cp_bn - sb : 0u)};
        if (++cp_kt == nk) {
            cp_kt = 0;
            cp_tile += gridDim.x;
            set_copy_tile();
        }
        return r;
    };
    if constexpr (PERS) set_copy_tile();

    // ---- per-lane LDS read offsets -------------------------------------------
    // A (second MFMA operand): lane l reads row wm*WM + bm*32 + l%32,
    // k = kk*16 + (l/32)*8 .. +7  (16-B chunk 2kk + l/32).  The swizzle depends on
    // the row's low 4 bits only, which are those of l%32.
    // (16x16x32: lane l reads row l%16, k = kk*32 + (l/16)*8 .. +7, chunk 4kk + l/16; the
    // swizzle depends on the row's low 4 bits, the same for every 16-row fragment)
    int aoff[KSTEPS];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
        const int c = MI == 32 ? kk * 2 + (lane >> 5) : kk * 4 + (lane >> 4);
        const int r = lane & (MI - 1);
        aoff[kk] = (wm * WM + r) * ROWB + (SWZ ? (c ^ kswz_t<BK>(r)) : c) * 16;
    }
    // B (first MFMA operand): lane l needs column n = wn*WN + bn*32 + l%32 with the
    // same 8 k values as A.
    int boff[B_NK ? KSTEPS : TN];
    if constexpr (B_NK) {
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
            const int c = MI == 32 ? kk * 2 + (lane >> 5) : kk * 4 + (lane >> 4);
            const int r = lane & (MI - 1);
            boff[kk] = (wn * WN + r) * ROWB + (SWZ ? (c ^ kswz_t<BK>(r)) : c) * 16;
        }
    } else {
        // ds_read_b64_tr_b16: in each 16-lane group, lane i supplies 8 B of row
        // (k0 + i/4) at columns (n0 + 4*(i%4)) .. +3 and receives column n0 + i of
        // rows k0..k0+3.  32x32x16: lanes 16-31 take columns +16, lanes 32-63 rows +8;
        // 16x16x32: each 16-lane group takes rows +8 (k 8(l/16) .. +7 of the step).
        constexpr int RB = BN * 2;
        const int kl = MI == 32 ? (lane >> 5) * 8 + ((lane & 15) >> 2) : (lane >> 4) * 8 + ((lane & 15) >> 2);
#pragma unroll
        for (int bn = 0; bn < TN; ++bn) {
            const int chunk = MI == 32 ? (wn * WN + bn * 32) / 8 + ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1)
                                       : (wn * WN + bn * 16) / 8 + ((lane >> 1) & 1);
            boff[bn] = kl * RB + (SWZ ? (chunk ^ nswz(kl)) : chunk) * 16 + (lane & 1) * 8;
        }
    }

    using AccV = std::conditional_t<MI == 32, floatx16, floatx4>;
    constexpr int NACC = MI == 32 ? 16 : 4;   // accumulators per lane and MFMA tile
    AccV acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < NACC; ++e) acc[i][j][e] = 0.0f;
    auto mfma_step = [&](const u32x4& b, const u32x4& a, AccV& c) __attribute__((always_inline)) {
        if constexpr (MI == 32) c = mfma<BF16>(b, a, c);
        else c = mfma16<BF16>(b, a, c);
    };

    // ---- persistent: the compute side of the k-tile stream ----------------------
    // (c_tile, c_kt): the tile and k-tile the MFMAs are on.  A tile's epilogue stages
    // through pstg, 32 rows x WN outputs per wave, apart from the ring.
    int c_tile = blockIdx.x, c_kt = 0;
    __shared__ __attribute__((aligned(1024))) char pstg[PERS ? G::NW * 32 * WN * 2 : 16];
    auto pers_epilogue = [&](auto tile) __attribute__((always_inline)) {
        int etm, etn;
        tile_of(tile, args, etm, etn);
        char* stg = pstg + wave * (32 * WN * 2);
        const int mb = etm * BM + wm * WM, nb = etn * BN + wn * WN;
        const int ep = args.epilogue;
        auto store_as = [&](auto odc) __attribute__((always_inline)) {
            constexpr int OD = decltype(odc)::value;
            if (ep == kEpiGelu) store_tile<OD, kEpiGelu, TM, TN, WN>(acc, stg, args, mb, nb, lane);
            else if (ep == kEpiRelu) store_tile<OD, kEpiRelu, TM, TN, WN>(acc, stg, args, mb, nb, lane);
            else store_tile<OD, kEpiNone, TM, TN, WN>(acc, stg, args, mb, nb, lane);
        };
        if (args.out_dtype == kOutBF16) store_as(std::integral_constant<int, kOutBF16>{});
        else store_as(std::integral_constant<int, kOutF16>{});
    };

    // Operand fragments of one k-step (16 of K for 32x32x16, 32 for 16x16x32): A rows
    // (second MFMA operand) and B columns (first MFMA operand).  Two sets alternate so
    // that the LDS reads of step kk+1 are in flight while the MFMAs of step kk run.
    struct Frags {
        u32x4 a[TM];
        u32x4 b[TN];
    };
    // LDS read op r (compile-time) of stage kk into f: r < TM are the A rows, then
    // the B columns (one ds_read_b128 each for [N,K] storage, two transposing
    // reads -- k 0..3 and 4..7 of the lane's 8 -- for [K,N] storage).
    constexpr int NRD = TM + (B_NK ? TN : 2 * TN);
    auto read_op = [&](const Slot& slot, int kk, Frags& f, auto rc) __attribute__((always_inline)) {
        constexpr int r = decltype(rc)::value;
        if constexpr (r < TM) {
            f.a[r] = *(const SPG_LDS u32x4*)(slot.a + aoff[kk] + r * MI * ROWB);
        } else if constexpr (B_NK) {
            constexpr int bn = r - TM;
            f.b[bn] = *(const SPG_LDS u32x4*)(slot.b + boff[kk] + bn * MI * ROWB);
        } else {
            constexpr int bn = (r - TM) / 2, h = (r - TM) % 2;
            constexpr int RB = BN * 2;
            const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (SPG_LDS shortx4*)(slot.b + boff[bn] + (kk * G::KPS + h * 4) * RB));
            const u32x2 v2 = __builtin_bit_cast(u32x2, v);
            f.b[bn][2 * h] = v2[0];
            f.b[bn][2 * h + 1] = v2[1];
        }
    };
    auto load_frags = [&](const Slot& slot, int kk, Frags& f) __attribute__((always_inline)) {
        static_for<0, NRD>([&](auto rc) { read_op(slot, kk, f, rc); });
    };
    auto mma = [&](const Frags& f) __attribute__((always_inline)) {
#pragma unroll
        for (int bn = 0; bn < TN; ++bn)
#pragma unroll
            for (int bm = 0; bm < TM; ++bm)
                mfma_step(f.b[bn], f.a[bm], acc[bn][bm]);
    };
    // keep each stage's loads and MFMAs together: no motion across stage boundaries
    auto fence = []() __attribute__((always_inline)) {
        if constexpr (SCHED == 0) __builtin_amdgcn_sched_barrier(0);
    };

    constexpr int NMMA = TN * TM;
#ifndef SPG_READS_PER_STEP
#define SPG_READS_PER_STEP 2
#endif
    constexpr int RPS = SPG_READS_PER_STEP;  // LDS reads issued per MFMA step
    constexpr int CPS = G::L / KSTEPS;       // copy ops per stage when spread over a window
    static_assert(LDM == 0 || LDM == 4 || LDM == 5 || LDM == 6 || G::L % KSTEPS == 0, "copy ops must split evenly over the stages");
    // One MFMA stage with its memory traffic interleaved: step i issues MFMA i of
    // `now`, then copy op i and RPS LDS reads of the next stage (into `nx`, from
    // `rslot` at k-step rkk).  Copy modes: 1, all L direct-to-LDS ops of the k-tile
    // whose resources are `src`, into `cslot`, one every CSP steps (CSP = 2 where the
    // stage has at least twice as many MFMAs as copies, else 1: measured with 16x16x32
    // tiles at 8192^3, NN -2.5% and TN -1.3% time against one per step; a later start
    // or a spacing of 3 or 4 was slower); 2, register-staged ops J0 .. J0+CPS-1
    // (write the staged data into cslot, then load the k-tile of `src` into the
    // freed registers); 3, direct-to-LDS ops J0 .. J0+CPS-1.  Under the hand-placed
    // schedule (SCHED 0) a scheduling barrier after every step keeps this order, so
    // each wave hands the matrix pipe a new MFMA every step while the LDS and the
    // copies are fed in its shadow instead of in bursts; under the compiler-placed one
    // (SCHED 1) the same instructions are left to the compiler's scheduler.
    auto stage = [&](const Frags& now, const Slot& rslot, int rkk, Frags& nx,
                     const Slot& cslot, const auto& src, auto do_read, auto mode, auto j0c)
                     __attribute__((always_inline)) {
        constexpr bool RD = decltype(do_read)::value;
        constexpr int MD = decltype(mode)::value;
        constexpr int J0 = decltype(j0c)::value;
        constexpr int NCP = MD == 1 ? G::L / PF : (MD >= 2 ? CPS : 0);
        constexpr int CSP = (MD == 1 && NCP > 0 && NMMA >= 2 * NCP) ? 2 : 1;
        // LDS reads are front-loaded, RPS per step, so the last read of the stage has
        // most of the stage to return before the next stage's first MFMA needs it
        constexpr int NRS = (NRD + RPS - 1) / RPS;
        constexpr int STEPS = NMMA > NRS ? (NMMA > NCP ? NMMA : NCP) : (NRS > NCP ? NRS : NCP);
        static_for<0, STEPS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i < NMMA) {
                constexpr int bn = i / TM, bm = i % TM;
                mfma_step(now.b[bn], now.a[bm], acc[bn][bm]);
            }
            if constexpr (MD == 1 && i % CSP == 0 && i / CSP < NCP) {
                // the A-deep ring issues B before A, so that the wait before the next
                // barrier can leave A's copies in flight; the B-deep ring keeps the
                // order A, B and leaves B's
                constexpr int j = LDM == 4 ? (J0 + i / CSP + A_DMA) % G::L : J0 + i / CSP;
                dma_op(cslot, src, std::integral_constant<int, j>{}, NotFirst{});
            }
            if constexpr (MD == 2 && i < NCP) {
                lwrite_op(cslot, std::integral_constant<int, J0 + i>{}, NotFirst{});
                gload_op(src, std::integral_constant<int, J0 + i>{}, NotFirst{});
            }
            if constexpr (MD == 3 && i < NCP)
                dma_op(cslot, src, std::integral_constant<int, J0 + i>{}, NotFirst{});
            if constexpr (RD) {
                static_for<0, RPS>([&](auto rc) {
                    constexpr int r = i * RPS + decltype(rc)::value;
                    if constexpr (r < NRD) read_op(rslot, rkk, nx, std::integral_constant<int, r>{});
                });
            }
            fence();
        });
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    using M0_ = std::integral_constant<int, 0>;
    using M1_ = std::integral_constant<int, 1>;
    using M2_ = std::integral_constant<int, 2>;
    using M3_ = std::integral_constant<int, 3>;
    using Z_ = std::integral_constant<int, 0>;
    constexpr int kNoCopy = 0;

    // ---- the pipelined K loop ----------------------------------------------------
    //
    // One k-tile = KSTEPS MFMA stages (16 of K each with 32x32x16, 32 with 16x16x32).
    // Stage kk computes from fragment set kk % NF and reads the fragments of stage
    // kk+PF (of the next k-tile once that passes KSTEPS) into set (kk+PF) % NF.  The
    // one barrier of k-tile t sits before
    // stage KSTEPS-PF, just after this wave's last LDS read of slot t%S: once every
    // wave has passed it, (a) k-tile t+1, whose copies this wave has waited for, is
    // visible to all, and (b) nobody reads slot t%S any more, so it is released
    // and refilled with k-tile t+S while the last PF stages (whose MFMAs read
    // registers, not LDS) still run.  Those stages already read k-tile t+1, so the
    // matrix pipe has work across the k-tile boundary.
    //
    // Copies run in windows from one barrier to the next (KSTEPS stages: the last
    // PF of k-tile t and the first KSTEPS-PF of k-tile t+1).  The window that
    // starts at barrier t fills slot t%S with k-tile t+S: mode 0 issues all of its
    // copies in the window's first PF stages, modes 1 and 2 spread them, CPS per
    // stage (mode 1 writes the k-tile staged in VGPRs and loads the next one into
    // the freed registers).
    constexpr int NF = PF == 1 ? 2 : KSTEPS;   // fragment sets
    static_assert(KSTEPS % NF == 0, "fragment sets must tile the k-steps of a k-tile");
    Frags fr[NF];
    auto fset = [&](auto ic) -> Frags& { return fr[decltype(ic)::value % NF]; };
    constexpr bool DIRECT = LDM == 0 || LDM == 4 || LDM == 5 || LDM == 6;  // all copies of a window right after its barrier
    using ModeWin = std::integral_constant<int, DIRECT ? 1 : (REG ? 2 : 3)>;
    constexpr int WOPS = DIRECT ? G::L / PF : CPS;    // copy ops per window stage
    static_assert(!DIRECT || G::L % PF == 0, "copies must split over the lookahead stages");

    // stage kk of a k-tile: MFMAs of set kk, reads of step kk+PF from `cur` or `nxt`,
    // copies of window position `pos` (if any) from `src` into `cslot`
    auto kstage = [&](auto kc, const Slot& cur, const Slot& nxt, const Slot& cslot,
                      const auto& src, auto pos, auto do_read) __attribute__((always_inline)) {
        // Under the compiler-placed schedule each stage asks LLVM's instruction-group
        // scheduler for its interleaving strategy 2, which spreads the stage's LDS reads
        // evenly among its MFMAs instead of bunching them.  Measured interleaved against
        // the plain compiler schedule (B-deep ring, 16x16x32, B stored [K,N]): 8192^3
        // fp16 -0.8%, bf16 -0.9%, 6144x8192x8192 fp16 -0.8% time, bitwise equal results.
        if constexpr (SCHED == 1) __builtin_amdgcn_iglp_opt(2);
        constexpr int kk = decltype(kc)::value;
        constexpr int rk = kk + PF;
        constexpr int P = decltype(pos)::value;          // -1: no copies in this stage
        const Slot& rslot = rk < KSTEPS ? cur : nxt;
        using MD = std::integral_constant<int, P < 0 ? 0 : ModeWin::value>;
        using J = std::integral_constant<int, (P < 0 ? 0 : P) * WOPS>;
        stage(fset(kc), rslot, rk % KSTEPS, fset(std::integral_constant<int, rk>{}), cslot, src,
              do_read, MD{}, J{});
    };

    if constexpr (S == 1) {
        // the serial K loop: copy, wait, multiply, and only then let the next copy in
        const Slot r0 = slot_of(Z_{});
        const Slot none{nullptr, nullptr};
        issue(r0, 0, First{});
        for (int t = 0; t < nk; ++t) {
            wait_vmcnt<0>();
            __syncthreads();
            load_frags(r0, 0, fr[0]);
            static_for<0, KSTEPS>([&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                using RD = std::integral_constant<bool, kk + 1 < KSTEPS>;
                kstage(kc, r0, none, none, kNoCopy, std::integral_constant<int, -1>{}, RD{});
            });
            __syncthreads();
            poison_slot(r0);
            issue(r0, t + 1, NotFirst{});  // past the last k-tile: zeros
        }
    } else {
        // The loop runs a whole number of S-groups: k-tiles t >= nk are copied as
        // zeros (empty resources), so the extra MFMAs add exact zeros and the body
        // needs no branches.
        const int nt = ((nk + S - 1) / S) * S;
        auto first_of = [](auto sc) { return std::integral_constant<bool, decltype(sc)::value == 0>{}; };
        constexpr int PRE = DIRECT ? 0 : PF * CPS;  // ops of k-tile S-1 the window before k-tile 0 moves
        if constexpr (PERS) {
            // prologue: the first S k-tiles of the stream fill every slot
            static_for<0, S>([&](auto sc) {
                const DmaSrc src = next_copy();
                static_for<0, G::L>([&](auto jc) { dma_op(slot_of(sc), src, jc, NotFirst{}); });
            });
            wait_vmcnt<(S - 1) * G::L>();
        } else if constexpr (LDM == 4) {
            // prologue: k-tiles 0 and 1, and A of k-tile 2; wait for k-tile 0
            issue(deep_slot(Z_{}), 0, First{});
            issue(deep_slot(std::integral_constant<int, 1>{}), 1, NotFirst{});
            const DmaSrc src = dma_src(2);
            static_for<0, A_DMA>([&](auto jc) {
                dma_op(deep_slot(std::integral_constant<int, 2>{}), src, jc, NotFirst{});
            });
            wait_vmcnt<G::L + A_DMA>();
        } else if constexpr (LDM == 6) {
            // prologue: k-tiles 0 and 1, and B of k-tile 2; wait for k-tile 0
            issue(deep_slot(Z_{}), 0, First{});
            issue(deep_slot(std::integral_constant<int, 1>{}), 1, NotFirst{});
            const DmaSrc src = dma_src(2);
            static_for<A_DMA, G::L>([&](auto jc) {
                dma_op(deep_slot(std::integral_constant<int, 2>{}), src, jc, NotFirst{});
            });
            wait_vmcnt<G::L + B_DMA>();
        } else if constexpr (LDM == 5) {
            // prologue: k-tiles 0 .. S-2 (slot S-1 is filled by the first window); wait
            // for k-tile 0
            static_for<0, S - 1>([&](auto sc) { issue(slot_of(sc), sc.value, first_of(sc)); });
            wait_vmcnt<(S - 2) * G::L>();
        } else if constexpr (LDM == 0) {
            // prologue: k-tiles 0 .. S-1 fill every slot; wait for k-tile 0
            static_for<0, S>([&](auto sc) { issue(slot_of(sc), sc.value, first_of(sc)); });
            wait_vmcnt<(S - 1) * G::L>();
        } else if constexpr (LDM == 2) {
            // prologue: k-tiles 0 .. S-2 whole, and the copies of k-tile S-1 that the
            // window before k-tile 0 would have issued; wait for k-tile 0
            static_for<0, S - 1>([&](auto sc) { issue(slot_of(sc), sc.value, first_of(sc)); });
            const DmaSrc src = dma_src(S - 1);
            static_for<0, PRE>([&](auto jc) {
                dma_op(slot_of(std::integral_constant<int, S - 1>{}), src, jc, NotFirst{});
            });
            wait_vmcnt<(S - 2) * G::L + PRE>();
        } else {
            // prologue: k-tiles 0 .. S-2 written, k-tile S-1 staged, the part of it that
            // the window before k-tile 0 moves written, and k-tile S loaded in its place
            static_for<0, S - 1>([&](auto sc) {
                const RegSrc src = reg_src(sc.value);
                static_for<0, G::L>([&](auto jc) { gload_op(src, jc, first_of(sc)); });
                static_for<0, G::L>([&](auto jc) { lwrite_op(slot_of(sc), jc, first_of(sc)); });
            });
            const RegSrc src1 = reg_src(S - 1), src2 = reg_src(S);
            static_for<0, G::L>([&](auto jc) { gload_op(src1, jc, NotFirst{}); });
            static_for<0, PRE>([&](auto jc) {
                lwrite_op(slot_of(std::integral_constant<int, S - 1>{}), jc, NotFirst{});
                gload_op(src2, jc, NotFirst{});
            });
        }
        lds_barrier();
        // (the ping-pong schedule reads its first fragments in its first memory phase)
        if constexpr (SCHED != 2)
            static_for<0, PF>([&](auto kc) { load_frags(slot_of(Z_{}), kc.value, fset(kc)); });

        // outstanding copies allowed at the wait before barrier t: k-tiles t+2 .. t+S-1
        // (in the A-deep ring, A of k-tile t+2; in the B-deep ring, B of k-tile t+2)
        constexpr int STEADY = LDM == 4 ? A_DMA : LDM == 6 ? B_DMA : (LDM == 5 ? (S - 3) * G::L : (S - 2) * G::L);
        auto ktile = [&](auto sc, int t) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            // slots of k-tiles t-1, t, t+1 (s = t mod S, or t mod 6 in the deep rings)
            auto slot_at = [&](auto ic) -> Slot {
                if constexpr (LDM == 4 || LDM == 6) return deep_slot(std::integral_constant<int, decltype(ic)::value % 6>{});
                else return slot_of(std::integral_constant<int, decltype(ic)::value % S>{});
            };
            constexpr int NS = (LDM == 4 || LDM == 6) ? 6 : S;
            const Slot cur = slot_at(sc);
            const Slot prev = slot_at(std::integral_constant<int, (s + NS - 1) % NS>{});
            const Slot nxt = slot_at(std::integral_constant<int, (s + 1) % NS>{});
            auto src_of = [&](int kt) __attribute__((always_inline)) {
                if constexpr (REG) return reg_src(kt);
                else return dma_src(kt);
            };
            if constexpr (DIRECT) {
                // all copies of a window are issued right after its barrier
                static_for<0, KSTEPS - PF>([&](auto kc) {
                    kstage(kc, cur, nxt, prev, kNoCopy, std::integral_constant<int, -1>{}, T_{});
                });
            } else {
                // the window that started at barrier t-1: k-tile t+S-1 into prev
                // (register staging: write k-tile t+S-1, load k-tile t+S)
                const auto src = src_of(REG ? t + S : t + S - 1);
                static_for<0, KSTEPS - PF>([&](auto kc) {
                    constexpr int kk = decltype(kc)::value;
                    using Pos = std::integral_constant<int, PF + kk>;
                    kstage(kc, cur, nxt, prev, src, Pos{}, T_{});
                });
            }
            if constexpr (!REG) wait_vmcnt<STEADY>();
            // every wave has finished reading slot s (released) and the next k-tile is
            // complete in its slot
            lds_barrier();
            // The stages after the barrier run at raised wave priority: with two waves
            // per SIMD the one that passed the barrier first keeps the matrix pipe
            // while its partner is still in the barrier's wake (measured at 8192^3 with
            // 128x64 wave tiles: +1.7% with 32x32x16; +1.2% NN and +2.6% TN with
            // 16x16x32, where no raised priority, dropping it part-way through the stage
            // or raising it before the barrier instead were all slower).
            __builtin_amdgcn_s_setprio(1);
            // the poison build: the regions released here (released at the previous
            // barrier, with release delay 1) become NaN before their refill is issued
            poison_slot(LDM == 5 ? prev : cur);
            {
                // the window that starts here: k-tile t+S into cur
                // (register staging: write k-tile t+S, load k-tile t+S+1)
                const auto src = [&]() __attribute__((always_inline)) {
                    if constexpr (PERS) return next_copy();
                    else if constexpr (LDM == 4) return DmaSrc{dma_src(t + 3).a, dma_src(t + 2).b};
                    else if constexpr (LDM == 6) return DmaSrc{dma_src(t + 2).a, dma_src(t + 3).b};
                    else if constexpr (LDM == 5) return dma_src(t + S - 1);
                    else return src_of(REG ? t + S + 1 : t + S);
                }();
                // the slot refilled: the one released here, or (release delay 1) the one
                // released at the previous barrier
                const Slot fill = LDM == 5 ? prev : cur;
                static_for<KSTEPS - PF, KSTEPS>([&](auto kc) {
                    constexpr int kk = decltype(kc)::value;
                    using Pos = std::integral_constant<int, kk - (KSTEPS - PF)>;
                    kstage(kc, cur, nxt, fill, src, Pos{}, T_{});
                });
            }
            __builtin_amdgcn_s_setprio(0);
            if constexpr (PERS) {
                // the MFMAs of the tile's last k-tile are issued: store it, start the next
                if (++c_kt == nk) {
                    if (c_tile < T) pers_epilogue(c_tile);
                    c_kt = 0;
                    c_tile += gridDim.x;
#pragma unroll
                    for (int i = 0; i < TN; ++i)
#pragma unroll
                        for (int j = 0; j < TM; ++j)
#pragma unroll
                            for (int e = 0; e < NACC; ++e) acc[i][j][e] = 0.0f;
                }
            }
        };
        if constexpr (SCHED == 2) {
            // Ping-pong schedule.  A workgroup's waves are dealt to the 4 SIMDs in turn,
            // so waves w and w+4 share a SIMD; waves 0..3 form group 0, waves 4..7 group
            // 1.  Every wave alternates a memory phase -- the LDS reads of one k-step's
            // fragments, and in the first k-step of a k-tile its copies into the slots
            // the previous k-tile released -- with a matrix phase that issues that
            // k-step's 32 MFMAs and nothing else.  Group 1 runs one phase behind group 0
            // and a workgroup barrier ends every phase, so in each phase one wave of
            // every SIMD multiplies from registers while its partner reads and copies;
            // the multiplying wave never waits for the LDS.
            //
            // Phases are numbered from the end of the prologue.  Group 0 reads k-step j
            // in phase 2j and multiplies it in phase 2j+1, group 1 one phase later, so
            // k-tile u (k-steps 2u, 2u+1) is read in phases 4u .. 4u+3.  Each wave waits
            // for its reads (lgkmcnt(0)) before the barrier that ends a memory phase, so
            // k-tile u's slots are free once the barrier ending phase 4u+3 has passed.
            // The first memory phase of k-tile u+1 (phase 4u+4 or 4u+5) copies A of
            // k-tile u+2 and B of k-tile u+3 into them (the B-deep ring: A slots t % 2,
            // B slots t % 3).  k-tile u+2 is first read in phase 4u+8; before the barrier
            // that opens it each wave waits for its copies of A(u+2) and B(u+2), leaving
            // only B(u+3) in flight: group 0 at the end of its matrix phase 4u+7, group 1
            // at the end of its memory phase 4u+7.  Both groups pass the same number of
            // barriers: group 1 one extra before its first phase, group 0 one after its
            // last.
            static_assert(LDM == 6 && S == 2 && MI == 16 && PF == 1 && G::NW == 8,
                          "ping-pong: 8 waves of 16x16x32 tiles on the B-deep ring");
            const int grp = wave >> 2;
            // The scheduling barriers keep every MFMA inside its phase: MFMAs touch
            // registers only, and the compiler would otherwise move them across the asm
            // barrier into the memory phase.
            auto phase_barrier = []() __attribute__((always_inline)) {
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_barrier" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
            };
            Frags f;
            auto matrix_phase = [&]() __attribute__((always_inline)) {
                static_for<0, NMMA>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    mfma_step(f.b[i / TM], f.a[i % TM], acc[i / TM][i % TM]);
                });
            };
            auto ktile_pp = [&](auto ic, int u) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value;
                const Slot cur = deep_slot(std::integral_constant<int, i>{});
                const Slot prev = deep_slot(std::integral_constant<int, (i + 5) % 6>{});
                // k-step 2u: fragments, then (u >= 1) the copies of A(u+1), B(u+2)
                load_frags(cur, 0, f);
                if (u >= 1) {
                    poison_slot(prev);
                    const DmaSrc src{dma_src(u + 1).a, dma_src(u + 2).b};
                    static_for<0, G::L>([&](auto jc) { dma_op(prev, src, jc, NotFirst{}); });
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                phase_barrier();
                matrix_phase();
                phase_barrier();
                // k-step 2u+1; A(u+1) and B(u+1) complete before k-tile u+1 is read
                load_frags(cur, 1, f);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (grp == 1) wait_vmcnt<B_DMA>();
                phase_barrier();
                matrix_phase();
                if (grp == 0) wait_vmcnt<B_DMA>();
                phase_barrier();
            };
            if (grp == 1) phase_barrier();
            int t0 = 0;
            for (; t0 + 6 <= nk; t0 += 6) {
                static_for<0, 6>([&](auto sc) { ktile_pp(sc, t0 + decltype(sc)::value); });
            }
            const int rem = nk - t0;
            static_for<0, 5>([&](auto sc) {
                if (decltype(sc)::value < rem) ktile_pp(sc, t0 + decltype(sc)::value);
            });
            if (grp == 0) phase_barrier();
        } else if constexpr (PERS) {
            // this workgroup's tiles as one stream of k-tiles, in whole S-groups (the
            // k-tiles past its last tile are zeros and nothing is stored for them)
            const int mine = (T - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
            const int ns = ((mine * nk + S - 1) / S) * S;
            for (int t0 = 0; t0 < ns; t0 += S) {
                static_for<0, S>([&](auto sc) { ktile(sc, t0 + decltype(sc)::value); });
            }
        } else if constexpr (LDM == 4 || LDM == 6) {
            // six k-tiles per iteration (the slot pattern repeats every 6), then the
            // remaining nk % 6 one by one: no k-tile past nk is multiplied
            int t0 = 0;
            for (; t0 + 6 <= nk; t0 += 6) {
                static_for<0, 6>([&](auto sc) { ktile(sc, t0 + decltype(sc)::value); });
            }
            const int rem = nk - t0;
            static_for<0, 5>([&](auto sc) {
                if (decltype(sc)::value < rem) ktile(sc, t0 + decltype(sc)::value);
            });
        } else {
            for (int t0 = 0; t0 < nt; t0 += S) {
                static_for<0, S>([&](auto sc) { ktile(sc, t0 + decltype(sc)::value); });
            }
        }
    }

    // ---- epilogue ------------------------------------------------------------
    if constexpr (PERS) {
        // every tile is stored; the zero-fill copies past the stream must land
        // before the workgroup ends
        wait_vmcnt<0>();
    } else {
        // the loop leaves zero-fill copies of k-tiles >= nt in flight: let them land
        // before the ring is reused for staging
        wait_vmcnt<0>();
        if (args.store_direct && args.out_dtype != kOutF32) {
            store_direct16<TM, TN, MI>(acc, args, m0 + wm * WM, n0 + wn * WN, lane);
            return;
        }
        __syncthreads();  // the ring is drained and free for staging
        char* stg;
        {
            const int sl = wave % S;
            char* base = sl == 0 ? ring0 : sl == 1 ? ring1 : sl == 2 ? ring2 : sl == 3 ? ring3
                       : sl == 4 ? ring4 : ring5;
            stg = base + (wave / S) * G::STGW;
        }
        // one branch on the (uniform) output type and epilogue, outside all accumulator reads
        const int od = args.out_dtype;
        const int ep = args.epilogue;
        const int m_base = m0 + wm * WM, n_base = n0 + wn * WN;
        auto store_as = [&](auto odc) __attribute__((always_inline)) {
            constexpr int OD = decltype(odc)::value;
            // several blocks per round only for one wave per SIMD: with two, the partner
            // wave already covers the latency (measured: +1.2% with 4 waves, -0.4% with 8)
            constexpr int NB32 = TM * MI / 32;   // 32-row blocks of the wave tile
            constexpr int NP = G::NW > 4 ? 1 : blocks_per_round<NB32, WN, OD == kOutF32 ? 4 : 2>(G::STGW);
            if constexpr (MI == 32) {
                if (ep == kEpiGelu) store_tile<OD, kEpiGelu, TM, TN, WN, NP>(acc, stg, args, m_base, n_base, lane);
                else if (ep == kEpiRelu) store_tile<OD, kEpiRelu, TM, TN, WN, NP>(acc, stg, args, m_base, n_base, lane);
                else store_tile<OD, kEpiNone, TM, TN, WN, NP>(acc, stg, args, m_base, n_base, lane);
            } else {
                if (ep == kEpiGelu) store_tile16<OD, kEpiGelu, TM, TN, WN, NP>(acc, stg, args, m_base, n_base, lane);
                else if (ep == kEpiRelu) store_tile16<OD, kEpiRelu, TM, TN, WN, NP>(acc, stg, args, m_base, n_base, lane);
                else store_tile16<OD, kEpiNone, TM, TN, WN, NP>(acc, stg, args, m_base, n_base, lane);
            }
        };
        if (od == kOutF32) store_as(std::integral_constant<int, kOutF32>{});
        else if (od == kOutBF16) store_as(std::integral_constant<int, kOutBF16>{});
        else store_as(std::integral_constant<int, kOutF16>{});
    }
}

// ---------------------------------------------------------------------------
// wave-specialized variant: one producer wave, NC consumer waves
// ---------------------------------------------------------------------------
//
// The warp-specialized pipeline of the Mosaic GPU pipelining guide (its "warp
// specialization" section and second matmul example): one wave issues every
// copy of the ring, the other waves only read LDS and run MFMA, and per-slot
// counters in LDS take the place of the per-k-tile workgroup barrier:
//   full[s]  = 1 + the last k-tile whose copies into slot s have completed
//              (written by the producer after s_waitcnt vmcnt, release store);
//   freed[s] = how many times a consumer wave has finished reading slot s
//              (each consumer adds 1 after its last read of a k-tile, release).
// Consumers wait for full[t % S] >= t + 1 before reading k-tile t; the producer
// waits for freed[s] >= NC * (t / S) before copying k-tile t into slot s.
// Every wait is bounded (kSpinMax polls with s_sleep in between, ~0.1 s): if a
// counter never arrived the wave goes on with wrong data instead of hanging, and
// adds 1 to the device word args.wait_timeouts, which the host reads back
// (gemm_wait_timeouts), so a give-up is never silent.
// The register file allots every wave of a workgroup the same VGPRs, so the
// producer costs a consumer's worth of registers: with 128x64 consumer tiles
// (two waves per SIMD at most) the tile is 256x128, four consumers + one producer.
constexpr int kSpinMax = 1 << 21;

// Ordering is explicit rather than through acquire/release atomics (whose
// workgroup-scope lowering may wait for every outstanding copy): the producer
// waits with s_waitcnt vmcnt for the copies a counter announces before it
// stores the counter; a consumer waits with s_waitcnt lgkmcnt(0) for its reads
// before it adds to one.  The LDS executes one wave's operations in order, so
// reads issued after a counter load has returned see what the counter announced;
// the compiler fence keeps them after the loop.
// A wait that exhausts its polls counts itself in *timeouts (one lane of the wave, a
// device-scope atomic add: a vector memory instruction) and returns.
__device__ __forceinline__ void wait_at_least(uint32_t* p, uint32_t target, uint32_t* timeouts) {
    int it = 0;
    for (; it < kSpinMax; ++it) {
        if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) break;
        __builtin_amdgcn_s_sleep(2);
    }
    if (it == kSpinMax && (threadIdx.x & 63) == 0 && timeouts != nullptr)
        __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("" ::: "memory");
}

template <bool BF16, bool B_NK, int BM, int BN, int BK, int WM, int WN, int S>
struct WsGeom {
    static constexpr int WAVES_N = BN / WN;
    static constexpr int NC = (BM / WM) * WAVES_N;     // consumer waves
    static constexpr int NT = (NC + 1) * 64;           // + the producer wave
    static constexpr int TM = WM / 32, TN = WN / 32;
    static constexpr int KSTEPS = BK / 16;
    static constexpr int ROWB = BK * 2;
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int STAGE = A_BYTES + BN * BK * 2;
    static constexpr int A_OPS = A_BYTES / 1024;       // copy instructions of one k-tile
    static constexpr int L = STAGE / 1024;
    static constexpr int STG = 32 * WN * 4;
    static_assert(BK == 64, "k-tile of 64");
    static_assert(S >= 2 && S * STAGE <= 160 * 1024 - 64, "LDS budget");
    static_assert(L < 64, "vmcnt range");
    static_assert(NC * STG <= S * STAGE, "epilogue staging must fit the ring");
    static_assert(BN >= 128, "[K,N] swizzle needs 16 chunks per row");
};

template <bool BF16, bool B_NK, int BM, int BN, int BK, int WM, int WN, int S>
__global__ void __launch_bounds__((WsGeom<BF16, B_NK, BM, BN, BK, WM, WN, S>::NT))
ws_gemm(KArgs args) {
    using G = WsGeom<BF16, B_NK, BM, BN, BK, WM, WN, S>;
    constexpr int NC = G::NC, TM = G::TM, TN = G::TN, ROWB = G::ROWB, A_BYTES = G::A_BYTES;
    constexpr int L = G::L, A_OPS = G::A_OPS;
    constexpr int CPR_K = BK / 8, RPI_K = 64 / CPR_K;

    __shared__ __attribute__((aligned(1024))) char ring[S * G::STAGE];
    __shared__ uint32_t full[S];
    __shared__ uint32_t freed[S];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int tm, tn;
    tile_of(blockIdx.x, args, tm, tn);
    const int M = args.M, N = args.N, K = args.K;
    const int m0 = tm * BM, n0 = tn * BN;
    const int nk = (K + BK - 1) / BK;
    const int pad = (BK - K % BK) % BK;

    if (threadIdx.x < S) { full[threadIdx.x] = 0; freed[threadIdx.x] = 0; }
    if constexpr (kPoison) {
        // the poison build: every slot starts as NaN
        for (int o = threadIdx.x * 16; o < (int)sizeof ring; o += G::NT * 16)
            *(u32x4*)(ring + o) = u32x4{~0u, ~0u, ~0u, ~0u};
    }
    __syncthreads();

    SPG_LDS char* ring_l = (SPG_LDS char*)ring;
    auto slot = [&](int t) __attribute__((always_inline)) { return ring_l + (t % S) * G::STAGE; };

    floatx16 acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    const int wm = wave / G::WAVES_N, wn = wave % G::WAVES_N;

    if (wave == NC) {
        // ---- producer: every copy of the ring --------------------------------------
        const int a_rows = (M - m0) < BM ? (M - m0) : BM;
        const uint64_t a_base = (uint64_t)(uintptr_t)(args.A + (size_t)m0 * K);
        const uint32_t a_bytes = (uint32_t)a_rows * (uint32_t)K * 2u;
        uint64_t b_base;
        uint32_t b_bytes, b_kb;
        if constexpr (B_NK) {
            const int b_rows = (N - n0) < BN ? (N - n0) : BN;
            b_base = (uint64_t)(uintptr_t)(args.B + (size_t)n0 * K);
            b_bytes = (uint32_t)b_rows * (uint32_t)K * 2u;
            b_kb = 2u;
        } else {
            b_base = (uint64_t)(uintptr_t)(args.B + n0);
            b_bytes = (uint32_t)(((size_t)K * N - n0) * 2u);
            b_kb = 2u * (uint32_t)N;
        }
        auto rsrc = [&](uint64_t base, uint32_t bytes, uint32_t kb, int kt) {
            const int64_t shift = (int64_t)(kt * BK - pad) * (int64_t)kb;
            return make_rsrc((const void*)(uintptr_t)(base + (uint64_t)shift), bytes - (uint32_t)shift);
        };
        // per-lane offsets of copy op j (the same layout the pipelined kernel uses)
        uint32_t off[L];
        int kin[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            if (j < A_OPS || B_NK) {
                const int d = j < A_OPS ? j : j - A_OPS;
                const int r = d * RPI_K + lane / CPR_K;
                const int p = lane % CPR_K;
                const int c = p ^ kswz_t<BK>(r);
                off[j] = (uint32_t)r * (uint32_t)K * 2u + (uint32_t)c * 16u;
                kin[j] = c * 8;
            } else {
                constexpr int CPR = BN / 8, RP = 64 / CPR;
                const int d = j - A_OPS;
                const int r = d * RP + lane / CPR;
                const int p = lane % CPR;
                const int c = p ^ nswz(r);
                off[j] = n0 + c * 8 + 8 > N ? kOOB : (uint32_t)r * (uint32_t)N * 2u + (uint32_t)c * 16u;
                kin[j] = r;
            }
        }
        auto issue = [&](int t, bool first) __attribute__((always_inline)) {
            const i32x4 ra = rsrc(a_base, a_bytes, 2u, t), rb = rsrc(b_base, b_bytes, b_kb, t);
            SPG_LDS char* dst = slot(t);
#pragma unroll
            for (int j = 0; j < L; ++j) {
                const uint32_t o = first && kin[j] < pad ? kOOB : off[j];
                dma16(j < A_OPS ? ra : rb, dst + j * 1024, o);
            }
        };
        auto publish = [&](int t) __attribute__((always_inline)) {
            asm volatile("" ::: "memory");
            if (lane == 0)
                __hip_atomic_store(&full[t % S], (uint32_t)(t + 1), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        issue(0, true);
        for (int t = 1; t < nk; ++t) {
            if (t >= S) {
                wait_at_least(&freed[t % S], (uint32_t)(NC * (t / S)), args.wait_timeouts);
                if constexpr (kPoison) {
                    // the poison build: the slot every consumer has released becomes NaN,
                    // and that write lands before the copies that refill it are issued
                    SPG_LDS char* dst = slot(t);
#pragma unroll
                    for (int j = 0; j < L; ++j)
                        *(SPG_LDS u32x4*)(dst + j * 1024 + lane * 16) = u32x4{~0u, ~0u, ~0u, ~0u};
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                }
            }
            issue(t, false);
            wait_vmcnt<L>();      // k-tile t-1 has landed
            publish(t - 1);
        }
        wait_vmcnt<0>();
        publish(nk - 1);
    } else {
        // ---- consumers: LDS reads and MFMA only ---------------------------------------
        int aoff[G::KSTEPS];
#pragma unroll
        for (int kk = 0; kk < G::KSTEPS; ++kk) {
            const int c = kk * 2 + (lane >> 5), r = lane & 31;
            aoff[kk] = (wm * WM + r) * ROWB + (c ^ kswz_t<BK>(r)) * 16;
        }
        int boff[B_NK ? G::KSTEPS : TN];
        if constexpr (B_NK) {
#pragma unroll
            for (int kk = 0; kk < G::KSTEPS; ++kk) {
                const int c = kk * 2 + (lane >> 5), r = lane & 31;
                boff[kk] = A_BYTES + (wn * WN + r) * ROWB + (c ^ kswz_t<BK>(r)) * 16;
            }
        } else {
            constexpr int RB = BN * 2;
            const int kl = (lane >> 5) * 8 + ((lane & 15) >> 2);
#pragma unroll
            for (int bn = 0; bn < TN; ++bn) {
                const int chunk = (wn * WN + bn * 32) / 8 + ((lane >> 4) & 1) * 2 + ((lane >> 1) & 1);
                boff[bn] = A_BYTES + kl * RB + (chunk ^ nswz(kl)) * 16 + (lane & 1) * 8;
            }
        }
        struct Frags { u32x4 a[TM]; u32x4 b[TN]; };
        constexpr int NRD = TM + (B_NK ? TN : 2 * TN);
        auto read_op = [&](const SPG_LDS char* sl, int kk, Frags& f, auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            if constexpr (r < TM) {
                f.a[r] = *(const SPG_LDS u32x4*)(sl + aoff[kk] + r * 32 * ROWB);
            } else if constexpr (B_NK) {
                f.b[r - TM] = *(const SPG_LDS u32x4*)(sl + boff[kk] + (r - TM) * 32 * ROWB);
            } else {
                constexpr int bn = (r - TM) / 2, h = (r - TM) % 2, RB = BN * 2;
                const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (SPG_LDS shortx4*)(sl + boff[bn] + (kk * 16 + h * 4) * RB));
                const u32x2 v2 = __builtin_bit_cast(u32x2, v);
                f.b[bn][2 * h] = v2[0];
                f.b[bn][2 * h + 1] = v2[1];
            }
        };
        // one MFMA stage of `now` with the reads of the next stage spread over its steps
        auto stage = [&](const Frags& now, const SPG_LDS char* sl, int kk, Frags& nx) __attribute__((always_inline)) {
            constexpr int NMMA = TN * TM, RPS = 2;
            constexpr int STEPS = NMMA > (NRD + 1) / RPS ? NMMA : (NRD + 1) / RPS;
            static_for<0, STEPS>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i < NMMA)
                    acc[i / TM][i % TM] = mfma<BF16>(now.b[i / TM], now.a[i % TM], acc[i / TM][i % TM]);
                static_for<0, RPS>([&](auto rc) {
                    constexpr int r = i * RPS + decltype(rc)::value;
                    if constexpr (r < NRD) read_op(sl, kk, nx, std::integral_constant<int, r>{});
                });
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        Frags f0, f1;
        wait_at_least(&full[0], 1u, args.wait_timeouts);
        static_for<0, NRD>([&](auto rc) { read_op(slot(0), 0, f0, rc); });
        for (int t = 0; t < nk; ++t) {
            const SPG_LDS char* cur = slot(t);
            stage(f0, cur, 1, f1);
            stage(f1, cur, 2, f0);
            stage(f0, cur, 3, f1);
            // this wave's reads of slot t % S are all issued: once they have returned
            // the slot is free for the producer
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane == 0)
                __hip_atomic_fetch_add(&freed[t % S], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (t + 1 < nk) wait_at_least(&full[(t + 1) % S], (uint32_t)(t + 2), args.wait_timeouts);
            // reads the first step of k-tile t+1 (a stale slot after the last one: unused)
            stage(f1, slot(t + 1), 0, f0);
        }
    }

    // ---- epilogue (consumers), staging in the drained ring ----------------------------
    __syncthreads();
    if (wave < NC) {
        char* stg = ring + wave * G::STG;
        const int m_base = m0 + wm * WM, n_base = n0 + wn * WN;
        const int od = args.out_dtype, ep = args.epilogue;
        auto store_as = [&](auto odc) __attribute__((always_inline)) {
            constexpr int OD = decltype(odc)::value;
            if (ep == kEpiGelu) store_tile<OD, kEpiGelu, TM, TN, WN>(acc, stg, args, m_base, n_base, lane);
            else if (ep == kEpiRelu) store_tile<OD, kEpiRelu, TM, TN, WN>(acc, stg, args, m_base, n_base, lane);
            else store_tile<OD, kEpiNone, TM, TN, WN>(acc, stg, args, m_base, n_base, lane);
        };
        if (od == kOutF32) store_as(std::integral_constant<int, kOutF32>{});
        else if (od == kOutBF16) store_as(std::integral_constant<int, kOutBF16>{});
        else store_as(std::integral_constant<int, kOutF16>{});
    }
}

// ---------------------------------------------------------------------------
// simple kernel: any shape, any alignment, any K (including 0)
// ---------------------------------------------------------------------------

template <bool BF16, bool B_NK>
__global__ void __launch_bounds__(256) simple_gemm(KArgs a) {
    constexpr int T = 64, TK = 16;
    __shared__ float As[TK][T + 1];
    __shared__ float Bs[TK][T + 1];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
    const int M = a.M, N = a.N, K = a.K;
    float acc[4][4] = {};
    // 64-bit k: K may be as large as INT32_MAX, where k0 + TK would overflow an int
    for (int64_t k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + i * 256;
            const int r = e / TK, kk = e % TK;
            const int gm = m0 + r;
            const int64_t gk = k0 + kk;
            As[kk][r] = (gm < M && gk < K) ? bits_to_f32(a.A[(size_t)gm * K + gk], BF16) : 0.0f;
            const int kb = e / T, c = e % T;
            const int64_t gkb = k0 + kb;
            const int gn = n0 + c;
            float bv = 0.0f;
            if (gkb < K && gn < N)
                bv = bits_to_f32(B_NK ? a.B[(size_t)gn * K + gkb] : a.B[(size_t)gkb * N + gn], BF16);
            Bs[kb][c] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int gm = m0 + ty * 4 + i;
        if (gm >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int gn = n0 + tx * 4 + j;
            if (gn >= N) continue;
            const float v = epi_apply(acc[i][j], a.epilogue);
            const size_t o = (size_t)gm * N + gn;
            if (a.out_dtype == kOutF32) ((float*)a.C)[o] = v;
            else ((uint16_t*)a.C)[o] = f32_to_bits(v, a.out_dtype == kOutBF16);
        }
    }
}

}  // namespace spg
