// int8 x int8 -> int32 products of the layer on CDNA4 MFMA, with fused
// dequant epilogues (mini_trainer guide: integer forward and backward matrix
// products; OneTrainer PR #1681: int8 product of quantized activations and
// weights).
//
// One kernel template serves the three products.  C[i, j] = sum_t A(i, t) *
// B(j, t) where each operand is stored either with the contraction index
// contiguous ("row" operand: element (i, t) at base[i * ld + t]) or with the
// contraction index as the row ("km" operand: element (i, t) at base[t * ld +
// i]):
//   forward  A = qx  [M,K] row, B = qw [N,K] row          C = y  [M,N]
//   dX       A = qg1 [M,N] row, B = qw [N,K] km (t = n)   C = dx [M,K]
//   dW       A = qg2 [M,N] km,  B = qx [M,K] km (t = m)   C = dw [N,K]
//
// Tiles of BM x BN outputs (256 x 256) and kBK (128) contraction bytes per
// stage are copied straight from global memory into LDS by 16-byte buffer
// loads, in the layout they have in memory (XOR-swizzled at 16-byte
// granularity), through a ring of stages (two at 128 bytes, as many as fit in
// 160 KiB of LDS, at most four) so the next stage's loads are in flight while
// one is multiplied.  Fragments for v_mfma_i32_32x32x32_i8 are read with
// ds_read_b128 from a row operand and with two ds_read_b64_tr_b8 from a km
// operand: in each 16-lane group the transpose read hands lane i byte i & 7
// of the row addressed by lane 2e + (i >> 3) as its byte e, so pointing lane
// s at contraction row k0 + (s >> 1), column c0 + 8 (s & 1) gives lane i the
// eight contraction values of column c0 + i: the same lane -> (column, k)
// map as a row operand's 16-byte read.
//
// The epilogue dequantizes (and for dX may rotate) in the accumulator layout,
// then passes the values through the idle stage buffers so that global
// stores write whole row segments.
//
// Exactness: int32 accumulation of int8 products is exact for contractions up
// to 131,071 and does not depend on the order of k, so the placement of k
// inside a fragment only has to agree between A and B, which it does.  Longer
// contractions run in chunks whose int32 sums are combined in an int64
// workspace (the MODE_CHUNK kernel variant, launch_product_long).  With a
// workspace, the tiles of a grid's partial last round are split along the
// contraction and their int32 partial sums added by the last piece to finish
// (the MODE_SPLIT variant, split_plan); the sum is the same integer.
#include "common.hpp"
#include "launch.hpp"

namespace qlin {

namespace {

typedef int i32x2v __attribute__((ext_vector_type(2)));

struct GemmParams {
    const int8_t *a;
    const int8_t *b;
    int64_t lda, ldb, ldc;
    int R, S, T;                   // output rows, output cols, contraction
    const float *srow;
    const float *scol;
    const float *bias;
    void *out;
    int tiles_i, tiles_j;
    int had;          // EPI_ROWSCALE_HAD: rotation block (2 .. 128, power of two)
    float had_scale;  // fl32(1 / sqrt(had))
    // Contractions split into chunks: ws [R, S] int64 (row stride ldc) holds
    // the running sum.  ws_mode 0: none; 1: store this chunk's sums; 2: add
    // them; 3: the epilogue takes acc + ws (the last chunk).
    int64_t *ws;
    int ws_mode;
    // Balanced last round (MODE_SPLIT): work units [0, full) are whole tiles;
    // each tile after them is covered by 'split' units, each owning a range
    // of its contraction stages.  part holds one BM x BN block of int32
    // partial sums per such unit; count[u] counts the units of tail tile u
    // that have stored theirs (returned to zero by the last one).
    int full, split;
    int32_t *part;
    unsigned *count;
};

// ------------------------------------------------------------------ staging

// Buffer resource over a whole operand: every lane offset used below is
// either a valid byte offset (< 2^31 - 16 by the shape limits) or kOob, which
// the buffer range check turns into a zero fill of the lane's 16 LDS bytes.
constexpr uint32_t kOob = 0x7FFFFFF0u;
constexpr int kRsrcWord3 = 0x00020000;   // raw 32-bit buffer format
// Cache policy of buffer accesses that must be coherent across the XCDs'
// L2s (sc1, the device-scope bit).
constexpr int kCoherent = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const int8_t *base)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(base), (short)0, (int)kOob,
                                             kRsrcWord3);
}

typedef __attribute__((address_space(3))) int8_t lds_i8;

// One operand tile of ROWS output rows (or columns) by kBK (64 or 128)
// contraction bytes,
// copied straight from global memory into LDS by buffer loads (each wave
// instruction fills 1 KiB: lane l writes bytes 16 l .. 16 l + 15).
//
// Row operand: LDS [ROWS][kBK]; the 16-byte chunk holding contraction bytes
// 16 c .. of row r sits at position c ^ ((r >> 2) & 3) for kBK = 64 and
// c ^ ((r >> 1) & 7) for kBK = 128, so the 16 rows read together by a
// fragment load fall on 16 distinct bank groups.
// Km operand: LDS [kBK][ROWS]; chunk c (columns 16 c ..) of contraction row k
// sits at position c ^ (2 (k & 7)) (for ROWS >= 256), so the 8 rows read
// together by a transpose load (and the neighbouring chunk read by the next
// 16 lanes) fall on distinct bank groups.
template <int ROWS, bool KM, int NT, int kBK>
struct Operand {
    static constexpr int kBytes = ROWS * kBK;
    static constexpr int kLoads = kBytes / 16 / NT;      // 16-byte loads per lane per stage
    static_assert(kBytes % (16 * NT) == 0, "tile does not split evenly over the threads");
    static constexpr int kRowChunks = KM ? ROWS / 16 : kBK / 16;

    __device__ static __forceinline__ int swz(int row)
    {
        if constexpr (!KM)
            return kBK == 64 ? (row >> 2) & 3 : (row >> 1) & 7;
        else if constexpr (ROWS >= 256)
            return 2 * (row & 7);
        else
            return row & (ROWS / 16 - 1) & 7;
    }

    // Enqueue the loads of stage k0 into 'dst' (this thread's share).
    __device__ static __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int64_t ld, int i0,
                                                 int lim, int k0, int T, bool live, int8_t *dst)
    {
        const int lane = __lane_id();
        const int w = threadIdx.x / kWave;
#pragma unroll
        for (int p = 0; p < kLoads; p++) {
            const int slot = (p * (NT / kWave) + w) * kWave + lane;   // 16-byte LDS slot
            const int row = slot / kRowChunks;
            const int c = (slot % kRowChunks) ^ swz(row);
            int gi, gk;
            int64_t off;
            if constexpr (KM) {
                gk = k0 + row;
                gi = i0 + 16 * c;
                off = (int64_t)gk * ld + gi;
            } else {
                gi = i0 + row;
                gk = k0 + 16 * c;
                off = (int64_t)gi * ld + gk;
            }
            const uint32_t voff = (live && gi < lim && gk < T) ? (uint32_t)off : kOob;
            lds_i8 *wave_dst = (lds_i8 *)dst + (p * (NT / kWave) + w) * (kWave * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)wave_dst,
                                                     16, voff, 0, 0, 0);
        }
    }

    // Raw registers of one MFMA fragment while its LDS reads are in flight.
    struct Raw {
        i32x4 v;            // row operand: one 16-byte read
        i32x2v lo, hi;      // km operand: two transpose reads
    };

    // Start loading the MFMA fragment of the 32 rows (columns) starting at
    // 'r0' for contraction step kk (32 bytes): lane l gets row r0 + l % 32 and
    // contraction bytes 16 (l / 32) .. +15 of the step.  Km fragments are read
    // by inline asm so that the compiler does not order them behind the buffer
    // loads still filling other stages; their registers are valid only after
    // settle().
    __device__ static __forceinline__ void frag(const int8_t *lds, int r0, int kk, Raw &f)
    {
        const int lane = __lane_id();
        if constexpr (KM) {
            const int s = lane % 16;
            const int krow = kk * 32 + (lane / 32) * 16 + (s >> 1);
            const int chunk = (r0 + ((lane % 32) / 16) * 16) / 16;
            const uint32_t base = (uint32_t)(uintptr_t)(const lds_i8 *)lds;
            const uint32_t a0 = base + krow * ROWS + 16 * (chunk ^ swz(krow)) + 8 * (s & 1);
            const uint32_t a1 =
                base + (krow + 8) * ROWS + 16 * (chunk ^ swz(krow + 8)) + 8 * (s & 1);
            asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(f.lo) : "v"(a0));
            asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(f.hi) : "v"(a1));
        } else {
            const int row = r0 + lane % 32;
            const int c = kk * 2 + lane / 32;
            f.v = *reinterpret_cast<const i32x4 *>(lds + row * kBK + 16 * (c ^ swz(row)));
        }
    }

    // After an lgkmcnt(0) wait: ties the asm-loaded registers to the wait so no
    // use (or copy) of them is scheduled before it.
    __device__ static __forceinline__ void settle(Raw &f)
    {
        if constexpr (KM) {
            asm volatile("" : "+v"(f.lo));
            asm volatile("" : "+v"(f.hi));
        }
    }

    __device__ static __forceinline__ i32x4 value(const Raw &f)
    {
        if constexpr (KM)
            return i32x4{f.lo[0], f.lo[1], f.hi[0], f.hi[1]};
        else
            return f.v;
    }
};

// Pipeline depth: as many stages as fit in this workgroup's share of the
// 160 KiB of LDS (OCC workgroups per CU), at most 4.
template <int kStageBytes, int OCC>
constexpr int kStagesFor()
{
    return (160 * 1024 / OCC / kStageBytes) < 4 ? (160 * 1024 / OCC / kStageBytes) : 4;
}

__device__ __forceinline__ void wait_lgkmcnt0()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without a memory fence: a fence would also wait for the
// loads of later stages still in flight.  LDS writes of a stage are complete
// once the writing lane's own vmcnt wait has passed, which every lane does
// before arriving here; the clobber keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence()
{
    asm volatile("s_barrier" ::: "memory");
}

// Epilogues: raw int32; dequant by the output row's scale; forward dequant by
// row and column scales plus bias; row-scale dequant followed by the block
// Hadamard rotation of each output row (blocks of up to 128 columns, which
// needs a wave tile 128 columns wide).
enum { EPI_RAW = 0, EPI_ROWSCALE = 1, EPI_FWD = 2, EPI_ROWSCALE_HAD = 3 };

// Tile order: workgroups are dispatched round-robin over the 8 XCDs, so
// consecutive ids are first regrouped per XCD (each XCD gets a contiguous
// range of the first n tiles), then walked in groups of kGroup tile rows so
// that tiles running together share their A rows and B columns in that XCD's
// L2.
constexpr int kGroup = 8;

__device__ __forceinline__ int xcd_order(int pid, int n)
{
    const int q = n / 8, rem = n % 8;
    const int xcd = pid % 8, idx = pid / 8;
    return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

__device__ __forceinline__ void tile_at(int lin, int tiles_i, int tiles_j, int &ti, int &tj)
{
    const int per_group = kGroup * tiles_j;
    const int g = lin / per_group;
    const int first = g * kGroup;
    const int gsize = tiles_i - first < kGroup ? tiles_i - first : kGroup;
    const int in = lin % per_group;
    ti = first + in % gsize;
    tj = in / gsize;
}

// Compute units of the chip: each runs one workgroup of the 256 x 256 tile
// configuration at a time, so a grid runs in rounds of this many tiles.
constexpr int kRound = 256;
// Fewest contraction stages a piece of a split tile gets, most pieces per
// tile, and most pieces in a round of three-way splits.  Every piece past the
// first adds a 256 KiB partial that the last one must read, and a nearly full
// round of three-way pieces ran slower than two-way ones: measured best were
// three pieces for 36 tiles left (12000 x 5376 -> 7168 forward), two for 76
// (its dW) and two for 128 (dW of 8192 tokens, 4096 <-> 14336: -3% and -8%
// against no split).
constexpr int kMinPieceStages = 4;
constexpr int kMaxPieces = 3;
constexpr int kMaxThreeWayUnits = 128;

// ------------------------------------------------------------------- kernel

// Launch modes.  MODE_CHUNK: the launch is one chunk of a contraction longer
// than the int32 bound (ws_mode 1-3).  MODE_SPLIT: the tiles left over after
// the last whole round of the grid are split along the contraction (full,
// split, part, count).  Ordinary launches carry neither's code.
enum { MODE_PLAIN = 0, MODE_CHUNK = 1, MODE_SPLIT = 2 };

template <int BM, int BN, int WM, int WN, int kBK, int OCC, bool AKM, bool BKM, int EPI,
          int MODE>
__global__ __launch_bounds__(WM *WN * 64, OCC) void gemm_kernel(GemmParams p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int FM = BM / WM / 32;   // 32x32 blocks per wave along rows
    constexpr int FN = BN / WN / 32;
    constexpr int NK = kBK / 32;       // MFMA contraction steps per stage
    using OpA = Operand<BM, AKM, NT, kBK>;
    using OpB = Operand<BN, BKM, NT, kBK>;
    constexpr int kStage = OpA::kBytes + OpB::kBytes;
    constexpr int kStages = kStagesFor<kStage, OCC>();
    static_assert(kStages >= 2, "tile too large for the LDS share");
    constexpr int kLoads = OpA::kLoads + OpB::kLoads;     // per lane per stage
    __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * kStage];

    // Work unit -> tile and range of contraction stages [kb, kb + KT).
    const int KT_all = (p.T + kBK - 1) / kBK;
    int lin, kb = 0, KT = KT_all, tail = -1, piece = 0;
    if (MODE == MODE_SPLIT && (int)blockIdx.x >= p.full) {
        const int q = (int)blockIdx.x - p.full;
        tail = q / p.split;
        piece = q % p.split;
        lin = p.full + tail;
        kb = piece * KT_all / p.split;
        KT = (piece + 1) * KT_all / p.split - kb;
    } else {
        lin = xcd_order(blockIdx.x, MODE == MODE_SPLIT ? p.full : p.tiles_i * p.tiles_j);
    }
    int ti, tj;
    tile_at(lin, p.tiles_i, p.tiles_j, ti, tj);
    const int i0 = ti * BM, j0 = tj * BN;
    const int lane = __lane_id();
    const int w = threadIdx.x / kWave;
    const int wi = w / WN, wj = w % WN;

    // Row operands address rows from their tile start; km operands address
    // columns from their tile start and contraction rows from each stage.
    const int8_t *abase = AKM ? p.a + i0 : p.a + (int64_t)i0 * p.lda;
    const int8_t *bbase = BKM ? p.b + j0 : p.b + (int64_t)j0 * p.ldb;
    const int alim = p.R - i0, blim = p.S - j0;

    // Stage s of the unit (stage kb + s of the contraction) goes to buffer
    // s % kStages.  Stages past the end are issued as all-out-of-range loads
    // (zero fills of a buffer that is never read) so every iteration waits
    // for the same number of loads.
    auto issue = [&](int s) {
        const bool live = s < KT;
        const int k0 = live ? (kb + s) * kBK : 0;
        int8_t *dst = smem + (s % kStages) * kStage;
        const int8_t *ak = AKM ? abase + (int64_t)k0 * p.lda : abase;
        const int8_t *bk = BKM ? bbase + (int64_t)k0 * p.ldb : bbase;
        OpA::issue(make_rsrc(ak), p.lda, 0, alim, AKM ? 0 : k0, AKM ? p.T - k0 : p.T, live, dst);
        OpB::issue(make_rsrc(bk), p.ldb, 0, blim, BKM ? 0 : k0, BKM ? p.T - k0 : p.T, live,
                   dst + OpA::kBytes);
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
            acc[a][b] = i32x16{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // Fragment reads of contraction step kk of a stage (into fa, fb), their
    // wait, and the MFMAs of one step.
    auto load = [&](const int8_t *stage, int kk, typename OpA::Raw *fa, typename OpB::Raw *fb) {
        const int8_t *lb = stage + OpA::kBytes;
#pragma unroll
        for (int a = 0; a < FM; a++)
            OpA::frag(stage, wi * (BM / WM) + a * 32, kk, fa[a]);
#pragma unroll
        for (int b = 0; b < FN; b++)
            OpB::frag(lb, wj * (BN / WN) + b * 32, kk, fb[b]);
    };
    auto settle = [&](typename OpA::Raw *fa, typename OpB::Raw *fb) {
        wait_lgkmcnt0();
#pragma unroll
        for (int a = 0; a < FM; a++)
            OpA::settle(fa[a]);
#pragma unroll
        for (int b = 0; b < FN; b++)
            OpB::settle(fb[b]);
    };
    auto mma = [&](const typename OpA::Raw *fa, const typename OpB::Raw *fb) {
        i32x4 av[FM], bv[FN];
#pragma unroll
        for (int a = 0; a < FM; a++)
            av[a] = OpA::value(fa[a]);
#pragma unroll
        for (int b = 0; b < FN; b++)
            bv[b] = OpB::value(fb[b]);
#pragma unroll
        for (int a = 0; a < FM; a++)
#pragma unroll
            for (int b = 0; b < FN; b++)
                acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bv[b], av[a], acc[a][b], 0, 0, 0);
    };

    // Stage s lives in buffer s % kStages and is issued at the top of stage
    // s - kStages + 1, into the buffer that the barrier closing the previous
    // stage has freed (every wave had read that stage into registers).  The
    // fragment sets alternate: the reads of step kk + 1 are in flight while
    // the MFMAs of step kk run; the first step of the next stage is read right
    // after the barrier that ends this one.  sched_barrier(0) pins this order
    // and sched_group_barrier spreads the stage's buffer loads over the MFMAs
    // of the first step.
    typename OpA::Raw fa[2][FM];
    typename OpB::Raw fb[2][FN];
#pragma unroll
    for (int s = 0; s < kStages - 1; s++)
        issue(s);
    wait_vmcnt<(kStages - 2) * kLoads>();
    barrier_no_fence();
    load(smem, 0, fa[0], fb[0]);

    for (int kt = 0; kt < KT; kt++) {
        const int8_t *cur = smem + (kt % kStages) * kStage;
#pragma unroll
        for (int kk = 0; kk + 1 < NK; kk++) {
            settle(fa[kk & 1], fb[kk & 1]);
            load(cur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
            if (kk == 0)
                issue(kt + kStages - 1);
            mma(fa[kk & 1], fb[kk & 1]);
            if (kk == 0) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * (FM + FN), 0);
#pragma unroll
                for (int g = 0; g < kLoads; g++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, (FM * FN + kLoads - 1) / kLoads, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // Stage kt + 1 has landed once at most the loads of stages kt + 2 ..
        // kt + kStages - 1 are outstanding.
        wait_vmcnt<(kStages - 2) * kLoads>();
        settle(fa[(NK - 1) & 1], fb[(NK - 1) & 1]);
        barrier_no_fence();
        if (kt + 1 < KT)
            load(smem + ((kt + 1) % kStages) * kStage, 0, fa[0], fb[0]);
        __builtin_amdgcn_sched_barrier(0);
        mma(fa[(NK - 1) & 1], fb[(NK - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();

    // Epilogue.  The MFMA ran with B as its first operand, so each 32x32
    // block holds C transposed: lane l has output row l % 32 and, in register
    // 4 g + e, output column 8 g + 4 (l / 32) + e.
    typedef long long i64x2 __attribute__((ext_vector_type(2)));
    auto ws_at = [&](int i, int j) { return p.ws + (int64_t)i * p.ldc + j; };
    // Four consecutive int64 running sums of row i from column j, or zeros
    // when this is not the last chunk of a split contraction.
    auto ws4 = [&](bool ok, int i, int j, int64_t e[4]) {
        if (MODE == MODE_CHUNK && p.ws_mode == 3 && ok && j < p.S) {
            const i64x2 *w = reinterpret_cast<const i64x2 *>(ws_at(i, j));
            const i64x2 lo = w[0], hi = w[1];
            e[0] = lo[0]; e[1] = lo[1]; e[2] = hi[0]; e[3] = hi[1];
        } else {
            e[0] = e[1] = e[2] = e[3] = 0;
        }
    };
    // fl32 of the accumulator (plus the running sum of earlier chunks).
    auto tofloat = [&](int32_t c, int64_t e) {
        if constexpr (MODE == MODE_CHUNK)
            return p.ws_mode == 3 ? (float)((int64_t)c + e) : (float)c;
        else
            return (float)c;
    };
    if constexpr (MODE == MODE_SPLIT) {
        if (tail >= 0) {
            // Store this unit's int32 sums in register order (coalesced
            // 16-byte runs) and count its arrival; the last of the tile's
            // units to arrive adds the others' sums (exact: int32 addition of
            // bounded partials) and runs the epilogue.
            //
            // The partial sums cross XCDs, whose L2s are not coherent with
            // one another.  They are written and read with the device-scope
            // coherence bit (sc1: the bit a device-scope relaxed atomic access
            // carries), so they never sit in an L2 as stale or dirty lines;
            // each wave waits for its stores to complete before the barrier
            // that precedes the arrival count, and the reader's loads are
            // issued after it observes the count.  A device-scope fence would
            // do the same by writing back and invalidating whole L2s, which
            // stalls the chip while the rest of the grid is still storing
            // outputs.
            //
            // The arrival flag lives in the stage buffers, free once every
            // wave has passed the main loop's last barrier: a second LDS
            // object would make the compiler wait for each stage's
            // buffer-to-LDS loads before any LDS read.
            int *last_unit = reinterpret_cast<int *>(smem);
            // Unit o's sums: wave w's FM x FN x 4 16-byte slots per lane, the
            // wave's slots contiguous.  Buffer resources start at this wave's
            // run (so slot offsets are constants); an empty resource reads
            // zeros.
            constexpr int kSlots = FM * FN * 4;
            const int wave = __builtin_amdgcn_readfirstlane(w);
            auto part_rsrc = [&](int o) {
                const int32_t *base = p.part + ((int64_t)tail * p.split + o) * (BM * BN) +
                                      (int64_t)wave * kSlots * kWave * 4;
                return make_rsrc(reinterpret_cast<const int8_t *>(base));
            };
            const uint32_t lane_off = (uint32_t)lane * 16;
            const __amdgpu_buffer_rsrc_t mine = part_rsrc(piece);
#pragma unroll
            for (int a = 0; a < FM; a++)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        const int slot = (a * FN + b) * 4 + g;
                        const i32x16 &c = acc[a][b];
                        __builtin_amdgcn_raw_buffer_store_b128(
                            i32x4{c[4 * g], c[4 * g + 1], c[4 * g + 2], c[4 * g + 3]}, mine,
                            lane_off, slot * kWave * 16, kCoherent);
                    }
            wait_vmcnt<0>();
            __syncthreads();
            if (threadIdx.x == 0) {
                const unsigned arrived = atomicAdd(p.count + tail, 1u);
                *last_unit = arrived == (unsigned)(p.split - 1);
                if (*last_unit)
                    atomicExch(p.count + tail, 0u);
            }
            __syncthreads();
            const bool is_last = *last_unit;
            // Every wave has read the flag before any reuses the stage
            // buffers for the output.
            __syncthreads();
            if (!is_last)
                return;
            // The other pieces' sums (at most two: kMaxPieces is 3), read for
            // two accumulator blocks at a time: sixteen 16-byte loads per
            // lane in flight, so the whole combine takes FM * FN / 2 round
            // trips.  A missing second piece reads zeros through an empty
            // buffer resource.
            static_assert(kMaxPieces <= 3 && (FM * FN) % 2 == 0, "combine batch shape");
            const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<int32_t *>(p.part), (short)0, 0, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rs[2] = {
                part_rsrc((piece + 1) % p.split),
                p.split > 2 ? part_rsrc((piece + 2) % p.split) : none};
#pragma unroll
            for (int q = 0; q < FM * FN; q += 2) {
                i32x4 t[2][2][4];
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int u = 0; u < 2; u++)
#pragma unroll
                        for (int g = 0; g < 4; g++)
                            t[h][u][g] = __builtin_amdgcn_raw_buffer_load_b128(
                                rs[u], lane_off, ((q + h) * 4 + g) * kWave * 16, kCoherent);
#pragma unroll
                for (int h = 0; h < 2; h++)
#pragma unroll
                    for (int u = 0; u < 2; u++)
#pragma unroll
                        for (int g = 0; g < 4; g++)
#pragma unroll
                            for (int e = 0; e < 4; e++)
                                acc[(q + h) / FN][(q + h) % FN][4 * g + e] += t[h][u][g][e];
            }
        }
    }
    if constexpr (MODE == MODE_CHUNK && EPI != EPI_RAW) {
        if (p.ws_mode == 1 || p.ws_mode == 2) {
#pragma unroll
            for (int a = 0; a < FM; a++) {
                const int i = i0 + wi * (BM / WM) + a * 32 + lane % 32;
                if (i >= p.R)
                    continue;
#pragma unroll
                for (int b = 0; b < FN; b++) {
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        const int j = j0 + wj * (BN / WN) + b * 32 + 8 * g + 4 * (lane / 32);
                        if (j >= p.S)
                            continue;
                        i64x2 *w = reinterpret_cast<i64x2 *>(ws_at(i, j));
                        i64x2 lo = {acc[a][b][4 * g], acc[a][b][4 * g + 1]};
                        i64x2 hi = {acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]};
                        if (p.ws_mode == 2) {
                            lo = lo + w[0];
                            hi = hi + w[1];
                        }
                        w[0] = lo;
                        w[1] = hi;
                    }
                }
            }
            return;
        }
    }
    // Output values of row block a of this wave, as 32-bit patterns in the
    // accumulator layout: v[b][4 g + e] belongs to row i0 + wi RW + 32 a +
    // lane % 32 and column j0 + wj CW + 32 b + 8 g + 4 (lane / 32) + e.  Rows
    // and columns past the output give zeros (they are never stored).
    constexpr int RW = BM / WM, CW = BN / WN;
    auto row_values = [&](int a, uint32_t (&out)[FN][16]) {
        const int i = i0 + wi * RW + a * 32 + lane % 32;
        const bool row_ok = i < p.R;
        float rs = 0.0f;
        if constexpr (EPI != EPI_RAW)
            rs = row_ok ? p.srow[i] : 0.0f;
        if constexpr (EPI == EPI_ROWSCALE_HAD) {
            static_assert(FN == 4, "the rotating epilogue needs 128-column wave tiles");
            // Within the wave's 128 columns, column c = 32 b + 8 g + 4 h + e
            // with h = lane / 32: butterfly strides 1 and 2 pair registers e,
            // stride 4 pairs lane l with lane l ^ 32, strides 8 and 16 pair
            // registers g and strides 32 and 64 pair blocks b.  Stages run in
            // ascending stride, the lower element becoming lo + hi and the
            // upper lo - hi, then every element is scaled once: the same
            // operations, in the same order, as the separate rotation of the
            // dequantized row.  (Lanes l and l ^ 32 share the row, so a row
            // past the output is all zeros on both.)
            const bool upper = lane >= 32;
            float v[FN][16];
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    int64_t e[4];
                    ws4(row_ok, i, j0 + wj * CW + b * 32 + 8 * g + 4 * (lane / 32), e);
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        v[b][4 * g + r] = tofloat(acc[a][b][4 * g + r], e[r]) * rs;
                }
            auto pair = [](float &lo, float &hi) {
                const float x = lo, y = hi;
                lo = x + y;
                hi = x - y;
            };
            if (p.had > 1)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        pair(v[b][4 * g], v[b][4 * g + 1]);
                        pair(v[b][4 * g + 2], v[b][4 * g + 3]);
                    }
            if (p.had > 2)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int g = 0; g < 4; g++) {
                        pair(v[b][4 * g], v[b][4 * g + 2]);
                        pair(v[b][4 * g + 1], v[b][4 * g + 3]);
                    }
            if (p.had > 4)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        // v_permlane32_swap exchanges the upper half of its
                        // first operand with the lower half of its second:
                        // with both the same value, lane l finds lane
                        // l ^ 32's value in the second result (l < 32) or
                        // the first (l >= 32).
                        const uint32_t u = __float_as_uint(v[b][r]);
                        const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
                        const float o = __uint_as_float(upper ? sw[0] : sw[1]);
                        v[b][r] = upper ? o - v[b][r] : v[b][r] + o;
                    }
            if (p.had > 8)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        pair(v[b][e], v[b][4 + e]);
                        pair(v[b][8 + e], v[b][12 + e]);
                    }
            if (p.had > 16)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        pair(v[b][e], v[b][8 + e]);
                        pair(v[b][4 + e], v[b][12 + e]);
                    }
            if (p.had > 32)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    pair(v[0][r], v[1][r]);
                    pair(v[2][r], v[3][r]);
                }
            if (p.had > 64)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    pair(v[0][r], v[2][r]);
                    pair(v[1][r], v[3][r]);
                }
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    out[b][r] = __float_as_uint(v[b][r] * p.had_scale);
        } else {
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int j = j0 + wj * CW + b * 32 + 8 * g + 4 * (lane / 32);
                    const i32x16 &c = acc[a][b];
                    if constexpr (EPI == EPI_RAW) {
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            out[b][4 * g + e] = (uint32_t)c[4 * g + e];
                    } else {
                        const bool ok = row_ok && j < p.S;
                        int64_t w[4];
                        ws4(ok, i, j, w);
                        f32x4 v;
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            v[e] = tofloat(c[4 * g + e], w[e]) * rs;
                        if constexpr (EPI == EPI_FWD) {
                            const f32x4 cs = ok ? *reinterpret_cast<const f32x4 *>(p.scol + j)
                                                : f32x4{0, 0, 0, 0};
#pragma unroll
                            for (int e = 0; e < 4; e++)
                                v[e] = v[e] * cs[e];
                            if (p.bias) {
                                const f32x4 bj = ok ? *reinterpret_cast<const f32x4 *>(p.bias + j)
                                                    : f32x4{0, 0, 0, 0};
#pragma unroll
                                for (int e = 0; e < 4; e++)
                                    v[e] = v[e] + bj[e];
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; e++)
                            out[b][4 * g + e] = __float_as_uint(v[e]);
                    }
                }
        }
    };

    // Stores go through LDS so that each store instruction writes whole row
    // segments (16 lanes per 256 bytes) instead of 32 bytes of 32 rows: each
    // wave owns a 16 KiB slice of the (now idle) stage buffers and passes its
    // RW x CW values through it in passes of 4096 words.  Within a row the
    // 16-byte chunks are XOR-swizzled by the row, so both the column-wise
    // writes and the row-wise reads spread over the banks.
    constexpr int kChunks = CW / 4;                  // 16-byte chunks per row
    constexpr int kPassRows = 4096 / CW;             // rows per pass
    constexpr int kPassBlocks = kPassRows / 32;      // 32-row blocks per pass
    static_assert(kPassBlocks >= 1 && FM % kPassBlocks == 0, "staging pass shape");
    static_assert(kStages * kStage >= NT / kWave * 4096 * 4, "staging needs 16 KiB per wave");
    lds_i8 *stage_base = (lds_i8 *)smem + w * 4096 * 4;
    auto slot = [&](int row, int chunk) { return row * CW + ((chunk ^ (row & (kChunks - 1))) * 4); };
#pragma unroll
    for (int pass = 0; pass < FM / kPassBlocks; pass++) {
#pragma unroll
        for (int q = 0; q < kPassBlocks; q++) {
            const int a = pass * kPassBlocks + q;
            uint32_t v[FN][16];
            row_values(a, v);
            const int row = q * 32 + lane % 32;
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    const int chunk = b * 8 + 2 * g + lane / 32;
                    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                    *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(
                        stage_base + 4 * slot(row, chunk)) =
                        u32x4{v[b][4 * g], v[b][4 * g + 1], v[b][4 * g + 2], v[b][4 * g + 3]};
                }
        }
        wait_lgkmcnt0();
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const int s16 = k * kWave + lane;            // 16-byte slot of the pass
            const int row = s16 / kChunks, chunk = s16 % kChunks;
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            const u32x4 t = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                stage_base + 4 * slot(row, chunk));
            const int i = i0 + wi * RW + pass * kPassRows + row;
            const int j = j0 + wj * CW + chunk * 4;
            if (i < p.R && j < p.S)
                *reinterpret_cast<u32x4 *>(static_cast<uint32_t *>(p.out) + (int64_t)i * p.ldc +
                                           j) = t;
        }
        wait_lgkmcnt0();
    }
}

template <int BM, int BN, int WM, int WN, int BK, int OCC, bool AKM, bool BKM, int EPI>
void run_gemm(const GemmParams &p0, hipStream_t st)
{
    GemmParams p = p0;
    p.tiles_i = (p.R + BM - 1) / BM;
    p.tiles_j = (p.S + BN - 1) / BN;
    const int tiles = p.tiles_i * p.tiles_j;
    if (p.ws_mode != 0) {
        if constexpr (EPI != EPI_RAW)
            hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, BK, OCC, AKM, BKM, EPI, MODE_CHUNK>),
                               dim3(tiles), dim3(WM * WN * 64), 0, st, p);
    } else if (p.split >= 2) {
        const unsigned grid = (unsigned)(p.full + (tiles - p.full) * p.split);
        if constexpr (EPI != EPI_RAW)
            hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, BK, OCC, AKM, BKM, EPI, MODE_SPLIT>),
                               dim3(grid), dim3(WM * WN * 64), 0, st, p);
    } else {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, BK, OCC, AKM, BKM, EPI, MODE_PLAIN>),
                           dim3(tiles), dim3(WM * WN * 64), 0, st, p);
    }
}

// Forward product for M <= 16 (decode-like shapes): the weight is streamed
// once.  Each workgroup owns 16 output columns, i.e. 16 weight rows, whose
// bytes are copied into LDS in chunks of CHUNK per row by buffer-to-LDS
// loads: each wave instruction fetches 1 KiB of one row, so every access is
// a whole contiguous run and a whole chunk (16 rows) is in flight at once,
// with the next chunk's loads issued before the current one is multiplied.
// Grids of at most one workgroup per compute unit take 4096-byte chunks (128
// KiB of buffers); larger grids take 1024-byte chunks, so that four
// workgroups share a compute unit (measured at 4096 -> 4096 and 4096 ->
// 14336: 8.0 -> 6.0 us and 17.4 -> 16.0 us for one and four tokens).  Inside a
// row, 16-byte piece c sits at slot c ^ (row & 15), so the MFMA reads of 16
// rows at one offset fall on distinct banks.  The 4 waves split a chunk's 64
// steps of 64 bytes, one v_mfma_i32_16x16x64_i8 per step with A = the
// (zero-padded) 16 rows of qx, and combine their int32 partials through LDS.
// 16x16 accumulator layout: lane l, register r holds column l % 16 and row
// 4 * (l / 16) + r.
template <bool RAW, int CHUNK>
__global__ __launch_bounds__(256) void skinny_fwd_kernel(const int8_t *__restrict__ qx,
                                                         const float *__restrict__ sx,
                                                         const int8_t *__restrict__ qw,
                                                         const float *__restrict__ sw,
                                                         const float *__restrict__ bias, int M,
                                                         int N, int K, void *__restrict__ out)
{
    constexpr int kBuf = 16 * CHUNK;            // one chunk of the 16 rows
    constexpr int kSegs = CHUNK / 1024;         // 1 KiB segments per row
    constexpr int kPer = CHUNK / 256;           // loads (and MFMA steps) per wave
    // Two chunk buffers, then the partials of the 4 waves (one LDS object, so
    // reads of one buffer do not wait for the loads filling the other).
    __shared__ __attribute__((aligned(1024))) int8_t smem[2 * kBuf + 4 * kWave * 16];
    const int lane = __lane_id();
    const int w = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int col = lane % 16, g = lane / 16;
    const bool xok = col < M;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(qx);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(qw + (int64_t)n0 * K);
    const int chunks = (K + CHUNK - 1) / CHUNK;

    // Chunk kc into buffer b: wave w's instruction p fills 1 KiB of row
    // (kPer w + p) / kSegs (its segment (kPer w + p) % kSegs); lane l's slot of
    // that row is 64 segment + l and holds piece slot ^ (row & 15).
    auto issue = [&](int kc, int b) {
#pragma unroll
        for (int p = 0; p < kPer; p++) {
            const int idx = w * kPer + p;
            const int row = idx / kSegs, slot = (idx % kSegs) * 64 + lane;
            const int k = kc * CHUNK + (slot ^ (row & 15)) * 16;
            const uint32_t off = kc < chunks && k < K ? (uint32_t)(row * K + k) : kOob;
            lds_i8 *dst = (lds_i8 *)smem + b * kBuf + row * CHUNK + (idx % kSegs) * 1024;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (__attribute__((address_space(3))) void *)dst, 16, off, 0, 0, 0);
        }
    };

    i32x4 acc = {0, 0, 0, 0};
    issue(0, 0);
    for (int kc = 0; kc < chunks; kc++) {
        // This wave's steps of the chunk: x fragments from global memory
        // (the same few rows for every workgroup, so L2-resident); rows past
        // M and bytes past K read as zeros through the buffer range check.
        i32x4 av[kPer];
#pragma unroll
        for (int t = 0; t < kPer; t++) {
            const int k = kc * CHUNK + (w + 4 * t) * 64 + g * 16;
            const uint32_t off = xok && k < K ? (uint32_t)(col * K + k) : kOob;
            av[t] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        }
        // The next chunk's loads (past the last chunk they are all out of
        // range: zero fills of the idle buffer), then wait until only they
        // are outstanding.  The same instruction sequence every iteration
        // keeps the compiler from adding waits of its own.
        issue(kc + 1, (kc + 1) & 1);
        wait_vmcnt<kPer>();
        barrier_no_fence();
        const int8_t *buf = smem + (kc & 1) * kBuf;
#pragma unroll
        for (int t = 0; t < kPer; t++) {
            const int piece = (w + 4 * t) * 4 + g;
            const i32x4 bv = *reinterpret_cast<const i32x4 *>(
                buf + col * CHUNK + (piece ^ col) * 16);
            acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t], bv, acc, 0, 0, 0);
        }
        // Every wave has read this buffer (its MFMAs consumed the reads)
        // before the loads of chunk kc + 2 refill it; no fence, so the loads
        // of chunk kc + 1 stay in flight.
        barrier_no_fence();
    }
    wait_vmcnt<0>();    // the zero fills issued by the last iteration
    i32x4 *red = reinterpret_cast<i32x4 *>(smem + 2 * kBuf);
    red[w * kWave + lane] = acc;
    __syncthreads();
    if (w != 0)
        return;
    const i32x4 t = (red[lane] + red[kWave + lane]) + (red[2 * kWave + lane] + red[3 * kWave + lane]);
    const int n = n0 + col;
    float cs = 0.0f, bn = 0.0f;
    if (!RAW) {
        cs = sw[n];
        if (bias)
            bn = bias[n];
    }
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int m = 4 * g + r;
        if (m >= M)
            continue;
        if (RAW) {
            static_cast<int32_t *>(out)[(int64_t)m * N + n] = t[r];
        } else {
            float f = (float)t[r] * sx[m];
            f = f * cs;
            if (bias)
                f = f + bn;
            static_cast<float *>(out)[(int64_t)m * N + n] = f;
        }
    }
}

// Tile configuration of the three products: 256 x 256 outputs per
// workgroup, 8 waves each owning 128 x 64, 128 contraction bytes per stage
// (two stages in flight in 128 KiB of LDS).
template <bool AKM, bool BKM, int EPI>
void run_cfg(const GemmParams &p, hipStream_t st)
{
    run_gemm<256, 256, 2, 4, 128, 1, AKM, BKM, EPI>(p, st);
}

} // namespace

SplitPlan split_plan(int op, int64_t M, int64_t N, int64_t K)
{
    SplitPlan none{0, 0, 1};
    if (op == 0 && M <= 16)
        return none;    // weight-streaming kernel
    const int64_t R = op == 2 ? N : M, S = op == 0 ? N : K, T = op == 0 ? K : (op == 1 ? N : M);
    const int64_t tiles = ((R + 255) / 256) * ((S + 255) / 256);
    const int64_t full = tiles / kRound * kRound, tail = tiles - full;
    if (tail == 0)
        return none;
    int64_t split = kRound / tail;
    const int64_t by_len = ((T + 127) / 128) / kMinPieceStages;
    split = split < by_len ? split : by_len;
    split = split < kMaxPieces ? split : kMaxPieces;
    if (split == 3 && tail * split > kMaxThreeWayUnits)
        split = 2;
    if (split < 2)
        return none;
    return SplitPlan{(int)full, (int)tail, (int)split};
}

size_t split_ws_bytes(const SplitPlan &sp)
{
    if (sp.split < 2)
        return 0;
    return kSplitCountBytes + (size_t)sp.tail * sp.split * 256 * 256 * sizeof(int32_t);
}

void launch_product(const ProductArgs &a, hipStream_t st)
{
    GemmParams p{};
    p.out = a.out;
    p.srow = a.srow;
    p.scol = a.scol;
    p.bias = a.bias;
    p.ws = a.ws;
    p.ws_mode = a.ws_mode;
    p.split = 1;
    if (a.split_ws && !a.raw && a.ws_mode == 0) {
        const SplitPlan sp = split_plan(a.op, a.M, a.N, a.K);
        if (sp.split >= 2) {
            p.full = sp.full;
            p.split = sp.split;
            p.count = static_cast<unsigned *>(a.split_ws);
            p.part = reinterpret_cast<int32_t *>(static_cast<char *>(a.split_ws) +
                                                 kSplitCountBytes);
        }
    }
    if (a.op == 0) {
        if (a.M <= 16 && a.ws_mode == 0) {
            const unsigned grid = (unsigned)(a.N / 16);
            auto go = [&](auto kernel) {
                hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, st, a.a, a.srow, a.b,
                                   a.scol, a.bias, (int)a.M, (int)a.N, (int)a.K, a.out);
            };
            const bool wide = grid > (unsigned)kRound;
            if (a.raw)
                wide ? go(skinny_fwd_kernel<true, 1024>) : go(skinny_fwd_kernel<true, 4096>);
            else
                wide ? go(skinny_fwd_kernel<false, 1024>) : go(skinny_fwd_kernel<false, 4096>);
            return;
        }
        p.a = a.a; p.lda = a.K;
        p.b = a.b; p.ldb = a.K;
        p.R = (int)a.M; p.S = (int)a.N; p.T = (int)(a.t_len ? a.t_len : a.K); p.ldc = a.N;
        if (a.raw)
            run_cfg<false, false, EPI_RAW>(p, st);
        else
            run_cfg<false, false, EPI_FWD>(p, st);
    } else if (a.op == 1) {
        p.a = a.a; p.lda = a.N;
        p.b = a.b; p.ldb = a.K;
        p.R = (int)a.M; p.S = (int)a.K; p.T = (int)(a.t_len ? a.t_len : a.N); p.ldc = a.K;
        if (a.raw) {
            run_cfg<false, true, EPI_RAW>(p, st);
        } else if (a.had >= 2 && a.had <= 128) {
            // dX with the un-rotation in the epilogue: 64 x 128 wave tiles.
            p.had = a.had;
            p.had_scale = a.had_scale;
            run_gemm<256, 256, 4, 2, 128, 1, false, true, EPI_ROWSCALE_HAD>(p, st);
        } else {
            run_cfg<false, true, EPI_ROWSCALE>(p, st);
        }
    } else {
        p.a = a.a; p.lda = a.N;
        p.b = a.b; p.ldb = a.K;
        p.R = (int)a.N; p.S = (int)a.K; p.T = (int)(a.t_len ? a.t_len : a.M); p.ldc = a.K;
        if (a.raw)
            run_cfg<true, true, EPI_RAW>(p, st);
        else
            run_cfg<true, true, EPI_ROWSCALE>(p, st);
    }
}

// Products whose contraction exceeds the int32-exact bound: chunks of 1023
// stages (130,944 terms, within the bound) run as ordinary products on the
// operands' sub-ranges; the first stores its int32 sums into the int64
// workspace, the middle ones add theirs, and the last one's epilogue takes
// acc + workspace through the usual dequant (and rotation) arithmetic.
void launch_product_long(const ProductArgs &a, int64_t *ws, hipStream_t st)
{
    constexpr int64_t kChunk = 1023 * 128;
    const int64_t T = a.op == 0 ? a.K : (a.op == 1 ? a.N : a.M);
    for (int64_t k0 = 0; k0 < T; k0 += kChunk) {
        ProductArgs c = a;
        const int64_t len = T - k0 < kChunk ? T - k0 : kChunk;
        c.t_len = len;
        c.ws = ws;
        c.ws_mode = k0 == 0 ? 1 : (k0 + len >= T ? 3 : 2);
        if (a.op == 0) {
            c.a = a.a + k0;
            c.b = a.b + k0;
        } else if (a.op == 1) {
            c.a = a.a + k0;
            c.b = a.b + k0 * a.K;
        } else {
            c.a = a.a + k0 * a.N;
            c.b = a.b + k0 * a.K;
        }
        launch_product(c, st);
    }
}

} // namespace qlin
