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
// Tiles of 256 x 256 outputs and 128 contraction bytes per stage are copied
// straight from global memory into LDS by 16-byte buffer loads, in the layout
// they have in memory (XOR-swizzled at 16-byte granularity), through two LDS
// stages so the next stage's loads are in flight while one is multiplied.
// Fragments for v_mfma_i32_16x16x64_i8 are read with ds_read_b128 from a row
// operand and with two ds_read_b64_tr_b8 from a km operand: in each 16-lane
// group the transpose read hands lane i byte i & 7 of the row addressed by
// lane 2e + (i >> 3) as its byte e, so pointing lane s at contraction row
// k0 + (s >> 1), column c0 + 8 (s & 1) gives lane i the eight contraction
// values of column c0 + i: the same lane -> (column, k) map as a row
// operand's 16-byte read.
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
#include <utility>

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

// Buffer resource over an operand from a base at the stage's start (row
// operand: the tile's first row at the stage's first contraction byte; km
// operand: the stage's first contraction row at the tile's first column), so
// that each lane's offsets are the same in every stage: every lane offset
// used below is either a byte offset whose 16 bytes end at or below kOob,
// which product_addressable checks for each shape before a launch, or kOob
// itself, which the buffer range check turns into a zero fill of the lane's
// 16 LDS bytes.
constexpr uint32_t kOob = 0x7FFFFFF0u;
// Cache policy of buffer accesses that must be coherent across the XCDs'
// L2s (sc1, the device-scope bit).
constexpr int kCoherent = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const int8_t *base,
                                                          uint32_t records = kOob)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(base), (short)0, (int)records,
                                             kRsrcWord3);
}

// Bytes a km operand's stage resource covers: all of a full stage, the first
// trel contraction rows of a partial one (whose later rows then read zeros:
// a lane's offset is its row times ld plus a column offset below ld, both
// multiples of 16), nothing of a stage past the unit's end.  For every shape
// product_addressable admits, trel * ld < 2^32 (ld <= 2^30, and
// (min(T, 128) - 1) ld + 256 <= kOob), so 32-bit arithmetic holds it; the
// clamp keeps kOob past the extent.
__device__ __forceinline__ uint32_t km_records(bool live, bool full, int trel, int64_t ld)
{
    if (!live)
        return 0;
    if (full)
        return kOob;
    const uint32_t n = (uint32_t)trel * (uint32_t)ld;
    return n < kOob ? n : kOob;
}

typedef __attribute__((address_space(3))) int8_t lds_i8;

// One operand tile of ROWS output rows (or columns) by kBK = 128 contraction
// bytes, copied straight from global memory into LDS by buffer loads (each
// wave instruction fills 1 KiB: lane l writes bytes 16 l .. 16 l + 15).
//
// Row operand: LDS [ROWS][128]; the 16-byte chunk holding contraction bytes
// 16 c .. of row r sits at position c ^ ((r >> 1) & 7), so the 16 rows read
// together by a fragment load fall on 16 distinct bank groups.
// Km operand: LDS [128][ROWS = 256]; chunk c (columns 16 c ..) of contraction
// row k sits at position c ^ (2 (k & 7) | ((k >> 4) & 1)): the 8 rows read
// together by one 16-lane group of a transpose load fall on distinct bank
// groups, and so do those of the next group, which reads the same chunk 16
// contraction rows further on.
template <int ROWS, bool KM, int NT, int kBK>
struct Operand {
    static constexpr int kBytes = ROWS * kBK;
    static constexpr int kLoads = kBytes / 16 / NT;      // 16-byte loads per lane per stage
    static_assert(kBytes % (16 * NT) == 0, "tile does not split evenly over the threads");
    static constexpr int kRowChunks = KM ? ROWS / 16 : kBK / 16;
    static_assert(kBK == 128 && (!KM || ROWS == 256), "operand layout shape");

    __device__ static __forceinline__ int swz(int row)
    {
        if constexpr (KM)
            return 2 * (row & 7) | ((row >> 4) & 1);
        else
            return (row >> 1) & 7;
    }

    // Load p of this lane: its output row or column within the tile and its
    // contraction index within the stage.
    __device__ static __forceinline__ void lane_slot(int p, int w, int &gi, int &gk)
    {
        const int slot = (p * (NT / kWave) + w) * kWave + __lane_id();   // 16-byte LDS slot
        const int row = slot / kRowChunks;
        const int c = (slot % kRowChunks) ^ swz(row);
        gi = KM ? 16 * c : row;
        gk = KM ? row : 16 * c;
    }

    // Byte offset of load p from a stage's base (the stage's first
    // contraction row, or byte, of the tile), the same in every stage; kOob
    // when the load's row or column lies past lim.
    __device__ static __forceinline__ uint32_t lane_offset(int p, int w, int64_t ld, int lim)
    {
        int gi, gk;
        lane_slot(p, w, gi, gk);
        const int64_t off = KM ? (int64_t)gk * ld + gi : (int64_t)gi * ld + gk;
        return gi < lim ? (uint32_t)off : kOob;
    }

    // Enqueue loads P0 .. P1 - 1 of this thread's share of a stage through
    // the resource rs based at the stage, into 'dst'.  voff holds the lane
    // offsets (lane_offset); w is the wave index, uniform.  A full stage uses
    // them as they are; otherwise loads whose contraction index reaches trel,
    // the contraction left from the stage's start, or every load of a stage
    // past the unit's end (!live), read zeros.
    template <int P0 = 0, int P1 = kLoads>
    __device__ static __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs,
                                                 const uint32_t (&voff)[kLoads], int trel,
                                                 bool live, bool full, int w, int8_t *dst)
    {
        auto load = [&](int p, uint32_t off) {
            lds_i8 *wave_dst = (lds_i8 *)dst + (p * (NT / kWave) + w) * (kWave * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)wave_dst,
                                                     16, off, 0, 0, 0);
        };
        if (KM || full) {
            // (A km operand's resource already bounds a partial stage.)
#pragma unroll
            for (int p = P0; p < P1; p++)
                load(p, voff[p]);
        } else {
#pragma unroll
            for (int p = P0; p < P1; p++) {
                int gi, gk;
                lane_slot(p, w, gi, gk);
                load(p, live && gk < trel ? voff[p] : kOob);
            }
        }
    }

    // An MFMA fragment's registers while its LDS reads are in flight.
    struct Raw {
        i32x4 v;            // row operand: one 16-byte read
        i32x2v lo, hi;      // km operand: two transpose reads
    };

    // Fragment of rows (columns) r0 .. r0 + 15 for one 64-byte contraction
    // step of v_mfma_i32_16x16x64_i8: lane l holds row r0 + l % 16 and
    // contraction bytes 16 (l / 16) .. +15 of the step.  off() gives the
    // lane's LDS byte offset in a stage for step 0 (row operand: for step
    // kk); the fragment of step kk of a km operand is at + kStep and, for a
    // row operand, that of the 16-row block f rows further on at + f kBlock
    // (neither moves the swizzle).  A km fragment's second transpose read is
    // 8 contraction rows on.
    __device__ static __forceinline__ uint32_t off(int r0, int kk)
    {
        const int lane = __lane_id();
        if constexpr (KM) {
            const int s = lane % 16;
            const int krow = (lane / 16) * 16 + (s >> 1);
            return krow * ROWS + 16 * ((r0 / 16) ^ swz(krow)) + 8 * (s & 1);
        } else {
            const int row = r0 + lane % 16, c = kk * 4 + lane / 16;
            return row * kBK + 16 * (c ^ swz(row));
        }
    }
    static constexpr int kStep = KM ? 64 * ROWS : 0;
    static constexpr int kBlock = KM ? 0 : 16 * kBK;
    static constexpr int kReads = KM ? 2 : 1;            // LDS instructions per fragment

    // Issue the reads of one fragment at LDS address 'addr' plus the constant
    // OFF.  Inline asm keeps the compiler from ordering them behind the buffer
    // loads still filling the other stage; the registers are valid only after
    // an lgkmcnt wait and settle().
    template <int OFF>
    __device__ static __forceinline__ void frag(uint32_t addr, Raw &f)
    {
        static_assert(OFF >= 0 && OFF + (KM ? 8 * ROWS : 0) < 65536, "LDS read immediate");
        if constexpr (KM) {
            asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(f.lo) : "v"(addr), "n"(OFF));
            asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2"
                         : "=v"(f.hi)
                         : "v"(addr), "n"(OFF + 8 * ROWS));
        } else {
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f.v) : "v"(addr), "n"(OFF));
        }
    }

    // After the fragment's lgkmcnt wait: ties its registers to the wait so no
    // use (or copy) of them is scheduled before it.
    __device__ static __forceinline__ void settle(Raw &f)
    {
        if constexpr (KM) {
            asm volatile("" : "+v"(f.lo));
            asm volatile("" : "+v"(f.hi));
        } else {
            asm volatile("" : "+v"(f.v));
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
// Hadamard rotation of each output row (blocks of up to 128 columns).
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

// What this workgroup computes: output tile (ti, tj) over the contraction
// stages [kb, kb + KT) of kBK bytes; tail >= 0 marks piece 'piece' of split
// tail tile 'tail'.
struct WorkUnit {
    int ti, tj, kb, KT, tail, piece;
};

template <int MODE>
__device__ __forceinline__ WorkUnit work_unit(const GemmParams &p, int kBK)
{
    const int KT_all = (p.T + kBK - 1) / kBK;
    WorkUnit u{0, 0, 0, KT_all, -1, 0};
    int lin;
    if (MODE == MODE_SPLIT && (int)blockIdx.x >= p.full) {
        const int q = (int)blockIdx.x - p.full;
        u.tail = q / p.split;
        u.piece = q % p.split;
        lin = p.full + u.tail;
        u.kb = u.piece * KT_all / p.split;
        u.KT = (u.piece + 1) * KT_all / p.split - u.kb;
    } else {
        lin = xcd_order(blockIdx.x, MODE == MODE_SPLIT ? p.full : p.tiles_i * p.tiles_j);
    }
    tile_at(lin, p.tiles_i, p.tiles_j, u.ti, u.tj);
    return u;
}

// Balanced last round: store this unit's int32 sums and count its arrival;
// the last of the tile's units to arrive adds the others' sums (exact: int32
// addition of bounded partials) and returns true, every other unit false.
// Each lane holds kSlots 16-byte slots of sums: get(s) reads slot s,
// add(s, v) adds v into it.
//
// The partial sums cross XCDs, whose L2s are not coherent with one another.
// They are written and read with the device-scope coherence bit (sc1: the bit
// a device-scope relaxed atomic access carries), so they never sit in an L2
// as stale or dirty lines; each wave waits for its stores to complete before
// the barrier that precedes the arrival count, and the reader's loads are
// issued after it observes the count.  A device-scope fence would do the
// same by writing back and invalidating whole L2s, which stalls the chip
// while the rest of the grid is still storing outputs.
//
// The arrival flag lives in the stage buffers ('flag_lds'), free once every
// wave has passed the barrier after the main loop (by then no wave's loads
// into those buffers are still landing): a second LDS object would make
// the compiler wait for each stage's buffer-to-LDS loads before any LDS read.
template <int kSlots, int kTile, int kBatch, typename Get, typename Add>
__device__ __forceinline__ bool split_combine(const GemmParams &p, int tail, int piece,
                                              int *flag_lds, Get get, Add add)
{
    // Unit o's sums: wave w's kSlots 16-byte slots per lane, the wave's slots
    // contiguous.  Buffer resources start at this wave's run (so slot offsets
    // are constants); an empty resource reads zeros.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    auto part_rsrc = [&](int o) {
        const int32_t *base = p.part + ((int64_t)tail * p.split + o) * kTile +
                              (int64_t)wave * kSlots * kWave * 4;
        return make_rsrc(reinterpret_cast<const int8_t *>(base));
    };
    const uint32_t lane_off = (uint32_t)__lane_id() * 16;
    const __amdgpu_buffer_rsrc_t mine = part_rsrc(piece);
#pragma unroll
    for (int s = 0; s < kSlots; s++)
        __builtin_amdgcn_raw_buffer_store_b128(get(s), mine, lane_off, s * kWave * 16, kCoherent);
    wait_vmcnt<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned arrived = atomicAdd(p.count + tail, 1u);
        *flag_lds = arrived == (unsigned)(p.split - 1);
        if (*flag_lds)
            atomicExch(p.count + tail, 0u);
    }
    __syncthreads();
    const bool is_last = *flag_lds;
    // Every wave has read the flag before any reuses the stage buffers for
    // the output.
    __syncthreads();
    if (!is_last)
        return false;
    // The other pieces' sums (at most two: kMaxPieces is 3), read kBatch
    // slots at a time: 2 kBatch 16-byte loads per lane in flight, so the
    // whole combine takes kSlots / kBatch round trips.  A missing second
    // piece reads zeros through an empty buffer resource.
    static_assert(kMaxPieces <= 3 && kSlots % kBatch == 0, "combine batch shape");
    const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t *>(p.part), (short)0, 0, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rs[2] = {part_rsrc((piece + 1) % p.split),
                                          p.split > 2 ? part_rsrc((piece + 2) % p.split) : none};
#pragma unroll
    for (int q = 0; q < kSlots; q += kBatch) {
        i32x4 t[kBatch][2];
#pragma unroll
        for (int h = 0; h < kBatch; h++)
#pragma unroll
            for (int o = 0; o < 2; o++)
                t[h][o] = __builtin_amdgcn_raw_buffer_load_b128(rs[o], lane_off,
                                                                (q + h) * kWave * 16, kCoherent);
#pragma unroll
        for (int h = 0; h < kBatch; h++)
            add(q + h, t[h][0] + t[h][1]);
        // (Otherwise the scheduler hoists every batch's loads to the top.)
        __builtin_amdgcn_sched_barrier(0);
    }
    return true;
}

// Second half of a staged output pass: the wave's LDS slice 'stage' holds
// 4096 words, kPassRows = 4096 / CW rows of CW columns whose 16-byte chunks
// sit at stage_slot(row, chunk); each of 16 store instructions writes whole
// row segments (16 lanes per 256 bytes) to the output from (i, j).
template <int CW>
__device__ __forceinline__ int stage_slot(int row, int chunk)
{
    constexpr int kChunks = CW / 4;
    return row * CW + ((chunk ^ (row & (kChunks - 1))) * 4);
}

//
// PAIR: the last stage of a rotation whose blocks span this wave's columns and
// those of the wave whose slice is 'partner' (same rows, the other CW
// columns of each 2 CW-column block): every value v and its partner value w
// become fl(fl(v + w) * had_scale) in the lower wave of the pair and
// fl(fl(w - v) * had_scale) in the upper one.
template <int CW, bool PAIR = false, bool NTS = false>
__device__ __forceinline__ void store_pass(const GemmParams &p, const lds_i8 *stage, int i, int j,
                                           const lds_i8 *partner = nullptr, bool upper = false)
{
    constexpr int kChunks = CW / 4;
    constexpr int kRowsPer = kWave / kChunks;      // rows per store instruction
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
    const int lane = __lane_id();
    // Store k writes row k kRowsPer + r0, 16-byte chunk 'chunk' (the same for
    // every k): one column test, and the row address advances by a constant.
    const int r0 = lane / kChunks, chunk = lane % kChunks;
    const bool col_ok = j + chunk * 4 < p.S;
    uint32_t *dst = static_cast<uint32_t *>(p.out) + (int64_t)(i + r0) * p.ldc + j + chunk * 4;
    const int64_t step = (int64_t)kRowsPer * p.ldc;
    const float sign = upper ? -1.0f : 1.0f;
    wait_lgkmcnt0();
#pragma unroll
    for (int k0 = 0; k0 < 16; k0 += 8) {
        // Eight slots' reads in flight together; the empty asm pins them
        // here (otherwise each is sunk into its guarded store below and
        // waited for alone).
        u32x4 t[8], o[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const int at = 4 * stage_slot<CW>((k0 + k) * kRowsPer + r0, chunk);
            t[k] = *reinterpret_cast<lds_u32x4 *>(stage + at);
            if constexpr (PAIR)
                o[k] = *reinterpret_cast<lds_u32x4 *>(partner + at);
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
            asm volatile("" : "+v"(t[k]));
            if constexpr (PAIR)
                asm volatile("" : "+v"(o[k]));
        }
#pragma unroll
        for (int k = 0; k < 8; k++) {
            if constexpr (PAIR) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    // own + partner (lower wave) or partner - own (upper),
                    // rounded once: sign * own is exact.
                    const float v = __uint_as_float(t[k][e]), x = __uint_as_float(o[k][e]);
                    t[k][e] = __float_as_uint(__builtin_fmaf(sign, v, x) * p.had_scale);
                }
            }
            if (col_ok && i + (k0 + k) * kRowsPer + r0 < p.R) {
                if constexpr (NTS)
                    __builtin_nontemporal_store(t[k], reinterpret_cast<u32x4 *>(dst));
                else
                    *reinterpret_cast<u32x4 *>(dst) = t[k];
            }
            dst += step;
        }
    }
    wait_lgkmcnt0();
}

// The buffer-to-LDS loads of stage s of a work unit (contraction stage
// kb + s): row operands address rows from their tile start (abase, bbase),
// km operands columns from their tile start and contraction rows from the
// stage.  Stages past the unit's end (s >= KT) are issued as all-out-of-range
// loads: zero fills of a buffer that is never read, so every iteration waits
// for the same number of loads.  plan() is computed once per stage; issue()
// enqueues loads G0 .. G1 - 1 of the stage's OpA::kLoads + OpB::kLoads per
// lane (A's first).
template <typename OpA, typename OpB, bool AKM, bool BKM, int kBK>
struct StageLoads {
    __amdgpu_buffer_rsrc_t ra, rb;
    int trel;
    bool live, full;

    __device__ static __forceinline__ StageLoads plan(const GemmParams &p, const int8_t *abase,
                                                      const int8_t *bbase, int kb, int KT, int s)
    {
        StageLoads L;
        L.live = s < KT;
        const int k0 = L.live ? (kb + s) * kBK : 0;
        L.trel = p.T - k0;
        L.full = L.live && L.trel >= kBK;
        const int8_t *ak = AKM ? abase + (int64_t)k0 * p.lda : abase + k0;
        const int8_t *bk = BKM ? bbase + (int64_t)k0 * p.ldb : bbase + k0;
        L.ra = make_rsrc(ak, AKM ? km_records(L.live, L.full, L.trel, p.lda) : kOob);
        L.rb = make_rsrc(bk, BKM ? km_records(L.live, L.full, L.trel, p.ldb) : kOob);
        return L;
    }

    template <int G0, int G1>
    __device__ __forceinline__ void issue(const uint32_t (&voffA)[OpA::kLoads],
                                          const uint32_t (&voffB)[OpB::kLoads], int w,
                                          int8_t *dstA, int8_t *dstB) const
    {
        constexpr int nA = OpA::kLoads;
        if constexpr (G0 < nA)
            OpA::template issue<G0, (G1 < nA ? G1 : nA)>(ra, voffA, trel, live, full, w, dstA);
        if constexpr (G1 > nA)
            OpB::template issue<(G0 > nA ? G0 - nA : 0), G1 - nA>(rb, voffB, trel, live, full, w,
                                                                  dstB);
    }
};

// Write one 16-byte chunk of a staged pass.
template <int CW>
__device__ __forceinline__ void stage_put(lds_i8 *stage, int row, int chunk, uint32_t a, uint32_t b,
                                          uint32_t c, uint32_t d)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(
        stage + 4 * stage_slot<CW>(row, chunk)) = u32x4{a, b, c, d};
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N - 1, so that the index
// can feed immediate operands.
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F &f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

template <int N>
__device__ __forceinline__ void wait_lgkmcnt()
{
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

// Four consecutive int64 running sums of row i from column j when this is the
// last chunk of a contraction past the int32 bound, otherwise zeros.
template <int MODE>
__device__ __forceinline__ void ws4(const GemmParams &p, bool ok, int i, int j, int64_t e[4])
{
    typedef long long i64x2 __attribute__((ext_vector_type(2)));
    if (MODE == MODE_CHUNK && p.ws_mode == 3 && ok && j < p.S) {
        const i64x2 *w = reinterpret_cast<const i64x2 *>(p.ws + (int64_t)i * p.ldc + j);
        const i64x2 lo = w[0], hi = w[1];
        e[0] = lo[0]; e[1] = lo[1]; e[2] = hi[0]; e[3] = hi[1];
    } else {
        e[0] = e[1] = e[2] = e[3] = 0;
    }
}

// fl32 of an accumulator plus the running sum of earlier chunks.
template <int MODE>
__device__ __forceinline__ float tofloat(const GemmParams &p, int32_t c, int64_t e)
{
    if constexpr (MODE == MODE_CHUNK)
        return p.ws_mode == 3 ? (float)((int64_t)c + e) : (float)c;
    else
        return (float)c;
}

// The product kernel: 256 x 256 tiles, 8 waves of RW x CW = 128 x 64 outputs
// in FM x FN = 8 x 4 blocks of 16 x 16, 128 contraction bytes per stage in
// two LDS stages (two MFMA steps of 64 bytes each).  Per lane the 128 int32
// sums of the wave tile fill 128 registers.  Each block's two steps run back
// to back, so the second MFMA takes the sums the first one produced (with
// random operands the matrix cores sustain 0.86-0.87 of their peak in that
// order against 0.81 step by step, at the same board power).  The column
// blocks' fragments of both steps stay in registers for the whole stage;
// the row blocks' fragments (both steps) are read one row block ahead into
// a ring of two.  Every fragment read is issued by inline asm (constant
// offsets in the instruction) and waited for with an lgkmcnt that counts the
// reads issued after it.
//
// The B operand is the MFMA's first operand, so block (a, b) holds C
// transposed: lane l has output row 16 a + l % 16 and, in register e, output
// column 16 b + 4 (l / 16) + e.
template <int WM, int WN, bool AKM, bool BKM, int EPI, int MODE>
__global__ __launch_bounds__(WM *WN * 64, 1) void gemm_kernel(GemmParams p)
{
    constexpr int BM = 256, BN = 256, kBK = 128;
    constexpr int NT = WM * WN * kWave;
    constexpr int RW = BM / WM, CW = BN / WN;
    constexpr int FM = RW / 16, FN = CW / 16;
    constexpr int NK = kBK / 64;                 // MFMA steps per stage
    // Parts a stage's buffer-to-LDS loads are issued in (one load each), and
    // how far ahead each operand's loads run.  A contiguous operand's loads
    // (lead 1) are for the next stage, behind the MFMA pairs of row blocks
    // 0-1 (behind the first two pairs of row blocks 0-3 instead: 0.6-0.7%
    // slower steps).  A contraction-strided operand's loads (lead 2) are for
    // the stage after next, behind the last row block's pairs, into the
    // buffers whose reads have just passed the stage barrier: a whole stage
    // to land (dW 4-5% and dX 3% faster; lead 2 for contiguous operands made
    // the forward 2% slower).
    constexpr int kSpread = 8;
    constexpr int kLeadA = AKM ? 2 : 1, kLeadB = BKM ? 2 : 1;
    static_assert(NK == 2 && FM % 2 == 0 && kSpread <= FN * (FM - 1) && kSpread % FN == 0,
                  "fragment schedule shape");
    using OpA = Operand<BM, AKM, NT, kBK>;
    using OpB = Operand<BN, BKM, NT, kBK>;
    constexpr int kStage = OpA::kBytes + OpB::kBytes;
    constexpr int kLoads = OpA::kLoads + OpB::kLoads;
    static_assert(kLoads == kSpread, "one load per part");
    // Loads of each lead (A's first): n1 behind the pairs of row blocks 0-1
    // for the next stage, n2 behind the last row block's pairs for the stage
    // after next; part_of(lead, i) is the i-th of them.
    constexpr int n1 = (kLeadA == 1 ? OpA::kLoads : 0) + (kLeadB == 1 ? OpB::kLoads : 0);
    constexpr int n2 = kLoads - n1;
    static_assert((n1 == 0 || (2 * FN) % n1 == 0) && n2 % FN == 0, "load placement");
    constexpr auto part_of = [](int lead, int i) {
        const int a = kLeadA == lead ? OpA::kLoads : 0;
        return i < a ? i : OpA::kLoads + (i - a);
    };
    constexpr int cA = OpA::kReads, cB = OpB::kReads;
    __shared__ __attribute__((aligned(1024))) int8_t smem[2 * kStage];

    const WorkUnit u = work_unit<MODE>(p, kBK);
    const int kb = u.kb, KT = u.KT;
    const int i0 = u.ti * BM, j0 = u.tj * BN;
    const int lane = __lane_id();
    const int w = threadIdx.x / kWave;
    const int wi = w / WN, wj = w % WN;
    const int8_t *abase = AKM ? p.a + i0 : p.a + (int64_t)i0 * p.lda;
    const int8_t *bbase = BKM ? p.b + j0 : p.b + (int64_t)j0 * p.ldb;
    const int alim = p.R - i0, blim = p.S - j0;
    // The lanes' load offsets within a stage, the same for every stage.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint32_t voffA[OpA::kLoads], voffB[OpB::kLoads];
#pragma unroll
    for (int q = 0; q < OpA::kLoads; q++)
        voffA[q] = OpA::lane_offset(q, wu, p.lda, alim);
#pragma unroll
    for (int q = 0; q < OpB::kLoads; q++)
        voffB[q] = OpB::lane_offset(q, wu, p.ldb, blim);
    // LDS holds the operands' stages operand by operand: A's two stages, then
    // B's, so that a stage's offset fits the LDS reads' immediate and the
    // unrolled loop below addresses either stage with constants.
    // Part G of stage s's buffer-to-LDS loads (planned in L), into buffers
    // s % 2.
    using Loads = StageLoads<OpA, OpB, AKM, BKM, kBK>;
    auto issue = [&](const Loads &L, int s, auto G) {
        constexpr int g = decltype(G)::value, per = kLoads / kSpread;
        L.template issue<g * per, (g + 1) * per>(voffA, voffB, wu, smem + (s & 1) * OpA::kBytes,
                                                 smem + 2 * OpA::kBytes + (s & 1) * OpB::kBytes);
    };

    // Lane offsets of this wave's fragments inside a stage: per step for a
    // row operand (blocks at constant offsets), per block for a km operand
    // (steps at constant offsets).
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_i8 *)smem;
    uint32_t offA[AKM ? FM : NK], offB[BKM ? FN : NK];
#pragma unroll
    for (int x = 0; x < (AKM ? FM : NK); x++)
        offA[x] = AKM ? OpA::off(wi * RW + 16 * x, 0) : OpA::off(wi * RW, x);
#pragma unroll
    for (int x = 0; x < (BKM ? FN : NK); x++)
        offB[x] = 2 * OpA::kBytes + (BKM ? OpB::off(wj * CW + 16 * x, 0) : OpB::off(wj * CW, x));

    i32x4 acc[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; a++)
#pragma unroll
        for (int b = 0; b < FN; b++)
            acc[a][b] = i32x4{0, 0, 0, 0};

    // Row block f's fragments of both steps in fa[f % 2][kk]; the column
    // blocks' fragments of both steps in fb[kk][b].
    typename OpA::Raw fa[2][NK];
    typename OpB::Raw fb[NK][FN];
    auto read_a = [&](auto P, auto F) {
        constexpr int f = decltype(F)::value, sl = f % 2;
        constexpr int st = decltype(P)::value * OpA::kBytes;
        static_for<NK>([&](auto KK) {
            constexpr int kk = decltype(KK)::value;
            if constexpr (AKM)
                OpA::template frag<st + kk * OpA::kStep>(lds0 + offA[f], fa[sl][kk]);
            else
                OpA::template frag<st + f * OpA::kBlock>(lds0 + offA[kk], fa[sl][kk]);
        });
    };
    auto read_b = [&](auto P, auto KK, auto Bi) {
        constexpr int kk = decltype(KK)::value, b = decltype(Bi)::value;
        constexpr int st = decltype(P)::value * OpB::kBytes;
        if constexpr (BKM)
            OpB::template frag<st + kk * OpB::kStep>(lds0 + offB[b], fb[kk][b]);
        else
            OpB::template frag<st + b * OpB::kBlock>(lds0 + offB[kk], fb[kk][b]);
    };
    auto read_b_pair = [&](auto P, auto Bi) {
        static_for<NK>([&](auto KK) { read_b(P, KK, Bi); });
    };
    // Block (f, b)'s two steps back to back: the second MFMA takes the sums
    // the first one produced.
    auto mfma_pair = [&](auto F, auto Bi) {
        constexpr int f = decltype(F)::value, b = decltype(Bi)::value, sl = f % 2;
#pragma unroll
        for (int kk = 0; kk < NK; kk++)
            acc[f][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                OpB::value(fb[kk][b]), OpA::value(fa[sl][kk]), acc[f][b], 0, 0, 0);
    };
    using Zero = std::integral_constant<int, 0>;
    using One = std::integral_constant<int, 1>;
    // Reads of a stage's head: row block 0, then the column blocks' pairs.
    auto head = [&](auto P) {
        read_a(P, Zero{});
        static_for<FN>([&](auto Bi) { read_b_pair(P, Bi); });
    };
    constexpr int rA = NK * cA, rB = NK * cB;       // LDS reads per row block, column block
    auto lgk = [](int n) { return n < 15 ? n : 15; };

    // Per stage: row block f's reads are issued one row block ahead, its
    // waits count the reads issued after them (LDS reads complete in order).
    // Row block 0 waits for each column block's pair just before its MFMAs:
    // those reads were issued behind the previous stage's last MFMAs.  Before
    // the last row block every read of the stage is waited for and the stage
    // barrier passes; the next stage's row block 0 is read, and each column
    // block's next pair is read into the registers that the last row block's
    // MFMA pair on that block has just used (an MFMA reads its A and B
    // operands when it issues, and only its sums, C, are read later; the LDS
    // read writes its registers when it returns).  Buffer-to-LDS loads go
    // out by their operand's lead (kLeadA, kLeadB).
    auto stage = [&](int kt, auto P) {
        constexpr int par = decltype(P)::value;
        const Loads L1 = Loads::plan(p, abase, bbase, kb, KT, kt + 1);
        const Loads L2 = Loads::plan(p, abase, bbase, kb, KT, kt + 2);
        static_for<FM - 1>([&](auto F) {
            constexpr int f = decltype(F)::value;
            read_a(P, std::integral_constant<int, f + 1>{});
            if constexpr (f > 0) {
                wait_lgkmcnt<lgk(rA)>();
#pragma unroll
                for (int kk = 0; kk < NK; kk++)
                    OpA::settle(fa[f % 2][kk]);
            }
            __builtin_amdgcn_sched_barrier(0);
            static_for<FN>([&](auto Bi) {
                constexpr int b = decltype(Bi)::value;
                if constexpr (f == 0) {
                    wait_lgkmcnt<lgk(rA + (FN - 1 - b) * rB)>();
                    if constexpr (b == 0) {
#pragma unroll
                        for (int kk = 0; kk < NK; kk++)
                            OpA::settle(fa[0][kk]);
                    }
#pragma unroll
                    for (int kk = 0; kk < NK; kk++)
                        OpB::settle(fb[kk][b]);
                }
                constexpr int slot = FN * f + b, every = 2 * FN / (n1 ? n1 : 2 * FN);
                if constexpr (n1 > 0 && slot < 2 * FN && slot % every == 0) {
                    issue(L1, kt + 1, std::integral_constant<int, part_of(1, slot / every)>{});
                    mfma_pair(F, Bi);
                    __builtin_amdgcn_sched_group_barrier(0x008, NK, 0);
                    __builtin_amdgcn_sched_group_barrier(0x020, kLoads / kSpread, 0);
                } else {
                    mfma_pair(F, Bi);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        // Stage kt + 1 has landed (its loads were the only ones in flight).
        wait_vmcnt<0>();
        wait_lgkmcnt<0>();
#pragma unroll
        for (int kk = 0; kk < NK; kk++)
            OpA::settle(fa[(FM - 1) % 2][kk]);
        barrier_no_fence();
        // (After the last stage these read the other buffer's stale bytes,
        // which no MFMA uses: no branch between the MFMAs.)
        read_a(std::integral_constant<int, 1 - par>{}, Zero{});
        __builtin_amdgcn_sched_barrier(0);
        static_for<FN>([&](auto Bi) {
            constexpr int b = decltype(Bi)::value;
            mfma_pair(std::integral_constant<int, FM - 1>{}, Bi);
            __builtin_amdgcn_sched_barrier(0);
            read_b_pair(std::integral_constant<int, 1 - par>{}, Bi);
            static_for<n2 / FN>([&](auto G) {
                issue(L2, kt + 2,
                      std::integral_constant<int, part_of(2, b * (n2 / FN) + decltype(G)::value)>{});
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    {
        const Loads L0 = Loads::plan(p, abase, bbase, kb, KT, 0);
        static_for<kSpread>([&](auto G) { issue(L0, 0, G); });
        const Loads L1 = Loads::plan(p, abase, bbase, kb, KT, 1);
        static_for<n2>([&](auto G) {
            issue(L1, 1, std::integral_constant<int, part_of(2, decltype(G)::value)>{});
        });
    }
    wait_vmcnt<n2>();       // stage 0 landed
    barrier_no_fence();
    head(Zero{});
    for (int kt = 0; kt < KT; kt += 2) {
        stage(kt, Zero{});
        if (kt + 1 < KT)
            stage(kt + 1, One{});
    }
    // The last stage has issued the next stage's fragment reads (never used)
    // and zero-fill loads into the stage buffers.  Wait for the reads and keep
    // their registers live through that wait: the compiler sees them written
    // at issue and would otherwise hand them to the code below while a read
    // is still in flight.  Then wait for this wave's loads, and barrier so
    // that no wave's loads are still landing when another wave writes its
    // staging slice (or its arrival flag) into the same buffers.
    wait_lgkmcnt<0>();
#pragma unroll
    for (int kk = 0; kk < NK; kk++) {
#pragma unroll
        for (int s = 0; s < 2; s++)
            OpA::settle(fa[s][kk]);
#pragma unroll
        for (int b = 0; b < FN; b++)
            OpB::settle(fb[kk][b]);
    }
    wait_vmcnt<0>();
    barrier_no_fence();

    if constexpr (MODE == MODE_SPLIT) {
        // Slot b + FN a of a lane holds block (a, b).
        if (u.tail >= 0 &&
            !split_combine<FM * FN, BM * BN, 8>(
                p, u.tail, u.piece, reinterpret_cast<int *>(smem),
                [&](int s) { return acc[s / FN][s % FN]; },
                [&](int s, i32x4 v) { acc[s / FN][s % FN] += v; }))
            return;
    }
    if constexpr (MODE == MODE_CHUNK) {
        // Not the last chunk: store (ws_mode 1) or add (2) the int32 sums
        // into the int64 running sums.
        if (p.ws_mode == 1 || p.ws_mode == 2) {
            typedef long long i64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int a = 0; a < FM; a++) {
                const int i = i0 + wi * RW + 16 * a + lane % 16;
#pragma unroll
                for (int b = 0; b < FN; b++) {
                    const int j = j0 + wj * CW + 16 * b + 4 * (lane / 16);
                    if (i >= p.R || j >= p.S)
                        continue;
                    i64x2 *ws = reinterpret_cast<i64x2 *>(p.ws + (int64_t)i * p.ldc + j);
                    i64x2 lo = {acc[a][b][0], acc[a][b][1]};
                    i64x2 hi = {acc[a][b][2], acc[a][b][3]};
                    if (p.ws_mode == 2) {
                        lo = lo + ws[0];
                        hi = hi + ws[1];
                    }
                    ws[0] = lo;
                    ws[1] = hi;
                }
                // (Otherwise every block's running sums are loaded at once.)
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
    }

    // Output values of row block a as 32-bit patterns, in the accumulator
    // layout: o[b][e] belongs to row i0 + wi RW + 16 a + l % 16 and column
    // j0 + wj CW + 16 b + 4 (l / 16) + e.  Rows and columns past the output
    // give zeros (they are never stored).  The forward product's column
    // scales and bias are the same for every row block.
    f32x4 cs[FN], bj[FN];
    if constexpr (EPI == EPI_FWD) {
#pragma unroll
        for (int b = 0; b < FN; b++) {
            const int j = j0 + wj * CW + 16 * b + 4 * (lane / 16);
            const bool ok = j < p.S;
            cs[b] = ok ? *reinterpret_cast<const f32x4 *>(p.scol + j) : f32x4{0, 0, 0, 0};
            bj[b] = ok && p.bias ? *reinterpret_cast<const f32x4 *>(p.bias + j)
                                 : f32x4{0, 0, 0, 0};
        }
    }
    // Row scales of every row block, loaded before the first store: on
    // gfx950 a load's vmcnt wait also waits for the stores issued before it.
    float rsv[FM];
#pragma unroll
    for (int a = 0; a < FM; a++) {
        const int i = i0 + wi * RW + 16 * a + lane % 16;
        rsv[a] = EPI != EPI_RAW && i < p.R ? p.srow[i] : 0.0f;
    }
    auto block_values = [&](int a, uint32_t (&o)[FN][4]) {
        const int i = i0 + wi * RW + 16 * a + lane % 16;
        const bool row_ok = i < p.R;
        const float rs = rsv[a];
        float v[FN][4];
#pragma unroll
        for (int b = 0; b < FN; b++) {
            if constexpr (EPI == EPI_RAW) {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    o[b][e] = (uint32_t)acc[a][b][e];
            } else {
                int64_t ext[4];
                ws4<MODE>(p, row_ok, i, j0 + wj * CW + 16 * b + 4 * (lane / 16), ext);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    v[b][e] = tofloat<MODE>(p, acc[a][b][e], ext[e]) * rs;
                    if constexpr (EPI == EPI_FWD) {
                        v[b][e] = v[b][e] * cs[b][e];
                        if (p.bias)
                            v[b][e] = v[b][e] + bj[b][e];
                    }
                }
            }
        }
        if constexpr (EPI == EPI_ROWSCALE_HAD) {
            static_assert(CW == 64, "the rotating epilogue is laid out for 64-column wave tiles");
            // Within a rotation block, column c = 64 (wj & 1) + 16 b + 4 h + e
            // with h = lane / 16: butterfly strides 1 and 2 pair registers e,
            // strides 4 and 8 pair lane l with lanes l ^ 16 and l ^ 32,
            // strides 16 and 32 pair blocks b, and stride 64 pairs the two
            // waves wj and wj ^ 1 (done in the store pass).  Stages run in
            // ascending stride, the lower element becoming lo + hi and the
            // upper lo - hi, then every element is scaled once: the same
            // operations, in the same order, as the separate rotation of the
            // dequantized row.  (The four lanes holding a row agree on
            // whether it is past the output, where all values are zero.)
            auto pair = [](float &lo, float &hi) {
                const float x = lo, y = hi;
                lo = x + y;
                hi = x - y;
            };
            if (p.had > 1)
#pragma unroll
                for (int b = 0; b < FN; b++) {
                    pair(v[b][0], v[b][1]);
                    pair(v[b][2], v[b][3]);
                }
            if (p.had > 2)
#pragma unroll
                for (int b = 0; b < FN; b++) {
                    pair(v[b][0], v[b][2]);
                    pair(v[b][1], v[b][3]);
                }
            // v_permlane16_swap exchanges the odd 16-lane rows of its first
            // operand with the even rows of its second, v_permlane32_swap the
            // upper half of its first with the lower half of its second: with
            // both operands the same value, every lane finds the lower
            // element of its pair (lo) in the first result and the upper
            // (hi) in the second.  lo + sign hi, with sign -1 in the upper
            // lanes, is computed as one fused multiply-add: sign hi is exact,
            // so it rounds once, exactly as lo + hi or lo - hi.
            if (p.had > 4) {
                const float sign = (lane / 16) & 1 ? -1.0f : 1.0f;
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const uint32_t x = __float_as_uint(v[b][e]);
                        const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
                        v[b][e] = __builtin_fmaf(sign, __uint_as_float(sw[1]),
                                                 __uint_as_float(sw[0]));
                    }
            }
            if (p.had > 8) {
                const float sign = lane >= 32 ? -1.0f : 1.0f;
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const uint32_t x = __float_as_uint(v[b][e]);
                        const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
                        v[b][e] = __builtin_fmaf(sign, __uint_as_float(sw[1]),
                                                 __uint_as_float(sw[0]));
                    }
            }
            if (p.had > 16)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    pair(v[0][e], v[1][e]);
                    pair(v[2][e], v[3][e]);
                }
            if (p.had > 32)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    pair(v[0][e], v[2][e]);
                    pair(v[1][e], v[3][e]);
                }
            if (p.had <= 64)
#pragma unroll
                for (int b = 0; b < FN; b++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        v[b][e] = v[b][e] * p.had_scale;
        }
        if constexpr (EPI != EPI_RAW) {
#pragma unroll
            for (int b = 0; b < FN; b++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    o[b][e] = __float_as_uint(v[b][e]);
        }
    };

    // Stores pass through the wave's 16 KiB slice of the idle stage buffers
    // (see store_pass), kPassRows rows at a time.  The forward and dX outputs
    // are stored non-temporally: nothing in a training step reads them again
    // soon, and stored through the 256 MB infinity cache they leave it full of
    // dirty lines that the next kernels' reads must first write back (the dY
    // statistics after the forward product, dW's operands after dX).  dW
    // stays cached: the weight update reads it next.
    constexpr bool kStream = EPI == EPI_FWD || EPI == EPI_ROWSCALE_HAD ||
                             (EPI == EPI_ROWSCALE && !AKM);
    constexpr int kPassRows = 4096 / CW;
    constexpr int kPassBlocks = kPassRows / 16;
    static_assert(FM % kPassBlocks == 0 && 2 * kStage >= NT / kWave * 4096 * 4, "staging shape");
    lds_i8 *stage_base = (lds_i8 *)smem + w * 4096 * 4;
#pragma unroll
    for (int pass = 0; pass < FM / kPassBlocks; pass++) {
#pragma unroll
        for (int q = 0; q < kPassBlocks; q++) {
            uint32_t o[FN][4];
            block_values(pass * kPassBlocks + q, o);
#pragma unroll
            for (int b = 0; b < FN; b++)
                stage_put<CW>(stage_base, 16 * q + lane % 16, 4 * b + lane / 16, o[b][0], o[b][1],
                              o[b][2], o[b][3]);
            // (The int64 sums of later blocks would be loaded here too, all
            // at once.)
            if constexpr (MODE == MODE_CHUNK)
                __builtin_amdgcn_sched_barrier(0);
        }
        const int i = i0 + wi * RW + pass * kPassRows, j = j0 + wj * CW;
        if (EPI == EPI_ROWSCALE_HAD && p.had > 64) {
            // Rotation blocks of 128 columns: wave pairs (wj, wj ^ 1) finish
            // the last stage through each other's slices, once both have
            // written them and before either overwrites its own.  The
            // barriers carry no fence, so the output stores stay in flight.
            wait_lgkmcnt0();
            barrier_no_fence();
            store_pass<CW, true, kStream>(p, stage_base, i, j, (lds_i8 *)smem + (w ^ 1) * 4096 * 4,
                                          wj & 1);
            barrier_no_fence();
        } else {
            store_pass<CW, false, kStream>(p, stage_base, i, j);
        }
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
        // (Only lanes of existing rows load: the others keep zeros.)
        i32x4 av[kPer];
#pragma unroll
        for (int t = 0; t < kPer; t++)
            av[t] = i32x4{0, 0, 0, 0};
        if (xok) {
#pragma unroll
            for (int t = 0; t < kPer; t++) {
                const int k = kc * CHUNK + (w + 4 * t) * 64 + g * 16;
                const uint32_t off = k < K ? (uint32_t)(col * K + k) : kOob;
                av[t] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
            }
        }
        // The next chunk's loads, then wait until only they are outstanding;
        // after the last chunk, for everything.  (Every wave issues the x
        // loads: each holds lanes of row 0.)
        if (kc + 1 < chunks) {
            issue(kc + 1, (kc + 1) & 1);
            wait_vmcnt<kPer>();
        } else {
            wait_vmcnt<0>();
        }
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

// Zero fill of n 32-bit words (arrival counters), a kernel rather than a
// memset so that it can sit in a captured graph.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int n)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n)
        p[i] = 0;
}

template <int WM, int WN, bool AKM, bool BKM, int EPI>
void run_gemm(const GemmParams &p0, hipStream_t st)
{
    GemmParams p = p0;
    p.tiles_i = (p.R + 255) / 256;
    p.tiles_j = (p.S + 255) / 256;
    const int tiles = p.tiles_i * p.tiles_j;
    const dim3 block(WM * WN * kWave);
    if (p.ws_mode != 0) {
        if constexpr (EPI != EPI_RAW)
            hipLaunchKernelGGL((gemm_kernel<WM, WN, AKM, BKM, EPI, MODE_CHUNK>), dim3(tiles), block,
                               0, st, p);
    } else if (p.split >= 2) {
        const unsigned grid = (unsigned)(p.full + (tiles - p.full) * p.split);
        if constexpr (EPI != EPI_RAW)
            hipLaunchKernelGGL((gemm_kernel<WM, WN, AKM, BKM, EPI, MODE_SPLIT>), dim3(grid), block,
                               0, st, p);
    } else {
        hipLaunchKernelGGL((gemm_kernel<WM, WN, AKM, BKM, EPI, MODE_PLAIN>), dim3(tiles), block, 0,
                           st, p);
    }
}

// Tile configuration of the three products: 256 x 256 outputs per
// workgroup, 8 waves each owning 128 x 64, 128 contraction bytes per stage
// (two stages in flight in 128 KiB of LDS).
template <bool AKM, bool BKM, int EPI>
void run_cfg(const GemmParams &p, hipStream_t st)
{
    run_gemm<2, 4, AKM, BKM, EPI>(p, st);
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

// Contraction terms per launch of a chunked product (1023 stages of 128):
// within the int32-exact bound of 131,071.
constexpr int64_t kChunkLen = 1023 * 128;

bool product_addressable(int op, int64_t M, int64_t N, int64_t K)
{
    const int64_t T = op == 0 ? K : (op == 1 ? N : M);
    const int64_t t = T > 131071 ? kChunkLen : T;       // contraction of one launch
    auto lo = [](int64_t a, int64_t b) { return a < b ? a : b; };
    // Row operand of 'rows' rows with stride ld: a tile's loads reach
    // (rows in the tile - 1) * ld + t bytes past its base.  Km operand with
    // stride ld: a stage's loads reach (contraction rows in the stage - 1) *
    // ld + 256 (one tile's columns).
    auto row_ok = [&](int64_t rows, int64_t ld) {
        return rows < 1 || (lo(rows, 256) - 1) * ld + t <= (int64_t)kOob;
    };
    auto km_ok = [&](int64_t ld) { return t < 1 || (lo(t, 128) - 1) * ld + 256 <= (int64_t)kOob; };
    if (op == 0)
        return row_ok(M, K) && row_ok(N, K);
    if (op == 1)
        return row_ok(M, N) && km_ok(K);
    return km_ok(N) && km_ok(K);
}

void launch_zero_words(void *p, int n, hipStream_t st)
{
    if (n > 0)
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                           static_cast<uint32_t *>(p), n);
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
            // dX with the un-rotation in the epilogue.
            p.had = a.had;
            p.had_scale = a.had_scale;
            run_cfg<false, true, EPI_ROWSCALE_HAD>(p, st);
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
    const int64_t T = a.op == 0 ? a.K : (a.op == 1 ? a.N : a.M);
    for (int64_t k0 = 0; k0 < T; k0 += kChunkLen) {
        ProductArgs c = a;
        const int64_t len = T - k0 < kChunkLen ? T - k0 : kChunkLen;
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
