// kernels_grouped.hip — grouped int8-MFMA expert GEMMs for large batches
// (prefill, T > 8).
//
// The same IDOT arithmetic as the GEMV path (colibri architecture overview,
// section 3.1: int4 weights dequantised on use, int8 activations, integer
// dot products), batched over the union of selected experts (colibri README
// zh-TW, "how it works": a batch reads each distinct expert once). Pairs
// (token, expert) are bucketed per expert and cut into tiles of 32 pairs.
//
// One wave computes a 32-row x 32-pair output tile. For every 32-wide block
// b it issues v_mfma_i32_32x32x32_i8 with
//   A = 32 weight rows x 32 k (lane l: row l%32, half l/32 holds 16 k),
//   B = 32 k x 32 pairs     (lane l: pair l%32, the same 16 k),
// unpacking the nibbles in registers (x16, exact), then adds
// C * (d_b/16) to an f64 accumulator per element: the block scale is per
// (token, block), so each block's int32 result is rescaled on its own.
// Both operands list their 16 k in the same order (the reordered 8-groups),
// so the product sums exactly the block's 32 k whatever order the matrix
// core uses inside a lane. Output element (row, pair) sits in lane
// pair + 32*((row/4)&1), register (row/8)*4 + row%4.
//
// The down kernels of the row-scale formats (int4, int2, int8) and their
// paired gate/up waves, in whole stages, swap the
// operands: pairs are the A rows and weight rows the B columns, so each
// group of four registers holds 8 pairs in every lane and a tile rescales
// only the groups its pairs fill (the pair-row form, at stage_pass_pr).
#include "device_common.hpp"
#include "internal.hpp"

namespace coli {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE_N = 32;     // pairs per tile (matches the bucket kernel)
constexpr int WAVES = 4;       // row tiles per workgroup

struct GroupedArgs {
    const uint8_t *q_a, *q_b;  // gate/up (both) or down (q_a)
    const float *s_a, *s_b;
    int H, I;
    const int8_t *act;         // gate/up: reordered Q8(x) [T][H]; down: reordered hq [pairs][I]
    const float *act_s;        // xs [T][H/32] or hs [pairs][I/32]
    const int *ctrl;
    const int2 *tiles;
    const int *expert_off, *pair_tok;
    float *h;
    int8_t *hq;
    float *hs;
    float *ye;
    int ntiles_max;            // tiles the grid covers
    int gsh;                   // group scales: log2(group / 32)
};

__device__ __forceinline__ v4i unpack8(uint2 w)
{
    const uint32_t m = 0xF0F0F0F0u;
    v4i a;
    a[0] = (int)((w.x << 4) & m);
    a[1] = (int)(w.x & m);
    a[2] = (int)((w.y << 4) & m);
    a[3] = (int)(w.y & m);
    return a;
}

__device__ __forceinline__ int tile_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

constexpr int N_XCD = 8;       // workgroups go round-robin over the 8 XCDs by index

// Tile-major order: with nrg a multiple of N_XCD, XCD x walks its row
// groups x, x + 8, ... for one tile before the next tile, so a tile's
// activation rows are read from memory once per XCD (then from its L2),
// and the tiles of one expert still follow each other, so each re-reads
// that expert's rows from the L2 a few workgroups after the one before.
__device__ __forceinline__ void tile_rg_tm(int w, int nrg, int ntiles, int &tile, int &rg)
{
    if (nrg % N_XCD == 0) {
        const int x = w % N_XCD, j = w / N_XCD, per = nrg / N_XCD;
        tile = j / per;
        rg = (j % per) * N_XCD + x;
    } else {
        tile = w / nrg;
        rg = w % nrg;
    }
}

// Keeps the loads above it issued before the work below it: without it the
// scheduler sinks a stage's loads to just before their use (to save
// registers), and every stage then waits out a full memory latency.
__device__ __forceinline__ void issue_fence() { __asm__ volatile("" ::: "memory"); }

// A pair of blocks (b, b+1): lane half h holds the 16 bytes of block b + h
// of its row, and one permlane32 swap per dword hands each half its 8 bytes
// of both blocks: afterwards A holds block b's bytes 8h..8h+7 and B block
// b+1's, the layout one MFMA per block expects.
__device__ __forceinline__ void split_pair(uint4 w, uint2 &A, uint2 &B)
{
    const auto s0 = __builtin_amdgcn_permlane32_swap(w.x, w.z, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(w.y, w.w, false, false);
    A = make_uint2(s0[0], s1[0]);
    B = make_uint2(s0[1], s1[1]);
}

// Staging. The K loop runs in stages of KS = 8 blocks: one 128-byte line of
// every weight row and 256 bytes of every pair's activation row. Global loads
// read whole lines (8 lanes per weight row, 16 lanes per activation row) into
// registers one stage ahead; after the current stage's MFMAs they go to LDS,
// from where each lane reads the pieces its MFMA operands need. The LDS
// serves a 16-byte access for 16 lanes per cycle across 64 banks (256
// bytes): weight row n's 16-byte chunk c sits at chunk position
// c ^ ((n >> 1) & 7) of its 128-byte row, pair p's chunk c at c ^ (p & 15)
// of its 256-byte row, so the 16 lanes of an access touch 16 different
// 16-byte bank groups both when storing lines and when reading columns.
// The weight rows of a wave are its own (single buffer); the activation
// rows are shared by the workgroup's waves (double buffer, one barrier per
// stage).
//
// int8 weights (WB = 8) store every block as two 16-byte halves, all first
// halves of a row and then all second halves (the activations' reordered
// 8-groups 0-1 and 2-3), and need no unpack. Their stages hold KS = 4
// blocks: a row's 8 LDS chunks are the 4 first halves, then the 4 second
// halves (two 64-byte runs of the row), and a pair's activations are 128
// bytes, whose chunk c sits at c ^ ((p >> 1) & 7) so that 16 pairs' reads of
// one column still touch 16 different bank groups.
//
// int2 weights (WB = 2) hold a 32-wide block in 8 bytes, one dword per 16
// columns, whose four 2-bit fields are the reordered activation dwords of
// those columns (byte k: columns 2k, 2k+1, 2k+8, 2k+9). Their stages hold
// KS = 8 blocks, 64 bytes of a row: 4 LDS chunks (chunk c: blocks 2c and
// 2c+1), at c ^ ((n >> 2) & 3); each lane loads one block.
//
// int4 codes with one f32 scale per group of columns (format code
// WB_GROUPS) stage 4 blocks (64 bytes of a row, each lane loading half a
// block), so that the group scales of a stage fit beside the tiles in LDS:
// four slots of 32 f64 scales per wave and matrix (slot k: the stage's k-th
// group; one slot when a group spans the stage).
constexpr int WB_GROUPS = 5;   // format code: int4 codes, a scale per group of columns
template <int WB> struct Stage;
template <> struct Stage<4> { static constexpr int KS = 8, WCH = 8; };
template <> struct Stage<8> { static constexpr int KS = 4, WCH = 8; };
template <> struct Stage<2> { static constexpr int KS = 8, WCH = 4; };
template <> struct Stage<WB_GROUPS> { static constexpr int KS = 4, WCH = 4; };
constexpr int GS_SLOTS = 4;    // group-scale slots per wave, matrix and stage

template <int WB> constexpr bool int4_codes() { return WB == 4 || WB == WB_GROUPS; }
template <int WB> constexpr int code_bits() { return WB == WB_GROUPS ? 4 : WB; }

template <int WB> constexpr int stage_blocks() { return Stage<WB>::KS; }
template <int WB> constexpr int stage_wch() { return Stage<WB>::WCH; }       // 16-byte weight chunks per row and stage
template <int WB> constexpr int stage_xc() { return 2 * Stage<WB>::KS; }   // 16-byte activation chunks per pair and stage

template <int WB> __device__ __forceinline__ int wsw(int n) { return stage_wch<WB>() == 4 ? ((n >> 2) & 3) : ((n >> 1) & 7); }
template <int WB> __device__ __forceinline__ int xsw(int p) { return stage_xc<WB>() == 16 ? (p & 15) : ((p >> 1) & 7); }

// Registers of one lane's share of a stage's weight loads: 16 bytes per
// load (int4, int8) or one 8-byte int2 block.
template <int WB> struct WReg { typedef v4i type; };
template <> struct WReg<2> { typedef v2i type; };
template <> struct WReg<WB_GROUPS> { typedef v2i type; };

// Staged data is held in clang vector types: plain loads and stores (copies
// of the HIP vector structs become memcpys that keep a stage in scratch).
typedef float v4f __attribute__((ext_vector_type(4)));

typedef double v2d __attribute__((ext_vector_type(2)));

template <int NM, int WB>
struct StageLds {
    v4i w[WAVES][NM][QK][stage_wch<WB>()];
    v4i x[2][TILE_N][stage_xc<WB>()];
    v2d d[2][stage_blocks<WB>() / 2][TILE_N];   // f64 block factors of the stage's block pairs (0 past the tile's pairs), pair-minor
    double sg[WB == WB_GROUPS ? WAVES : 1][NM][WB == WB_GROUPS ? GS_SLOTS : 1][WB == WB_GROUPS ? QK : 1];   // group scales, row-minor
};

__device__ __forceinline__ uint4 as_u4(v4i v) { return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]); }
__device__ __forceinline__ int4 as_i4(v4i v) { return make_int4(v[0], v[1], v[2], v[3]); }

// Loads of stage s. Rows past the matrix end are never touched (waves
// without rows skip the weight loads); blocks past nblk are clamped to the
// last block (their products are never added). Lane l loads chunk l % 8 of
// rows l/8, l/8 + 8, ...: int4, block l % 8 of the stage; int8, half
// (l % 8) / 4 of block l % 4 (rowb: bytes per row).
template <int WB>
__device__ __forceinline__ typename WReg<WB>::type load_w_row(int s, int nblk, const uint8_t *wrow, long rowb)
{
    typedef typename WReg<WB>::type R;
    constexpr int KS = stage_blocks<WB>();
    const int c = threadIdx.x & 7;
    const int blk = min(s * KS + (WB == 8 ? (c & 3) : WB == WB_GROUPS ? (c >> 1) : c), nblk - 1);
    const long off = WB == 4 ? 16 * blk
                   : WB == 2 ? 8 * blk
                   : WB == WB_GROUPS ? 16 * blk + 8 * (c & 1)
                   : (c >> 2) * (rowb / 2) + 16 * blk;
    return *reinterpret_cast<const R *>(wrow + off);
}

template <int WB>
__device__ __forceinline__ void load_w(typename WReg<WB>::type (&w)[4], int s, int nblk, const uint8_t *wrow, long rowb)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = load_w_row<WB>(s, nblk, wrow + (long)(8 * j) * rowb, rowb);
}

// Activation loads: 2 * KS lanes per pair row (16-byte chunk c of the
// stage: block c/2, half c%2), 64 / (2 * KS) pairs per load instruction.
template <int WB> constexpr int x_loads() { return stage_xc<WB>() / 8; }   // per wave and stage: 2 (int4), 1 (int8)

template <int WB>
__device__ __forceinline__ void load_x(v4i (&x)[x_loads<WB>()], int s, int nblk, const int8_t *const (&xrow)[x_loads<WB>()])
{
    constexpr int KS = stage_blocks<WB>(), XC = stage_xc<WB>();
    const int c = threadIdx.x & (XC - 1);
    const int xb = min(s * KS + (c >> 1), nblk - 1);
#pragma unroll
    for (int i = 0; i < x_loads<WB>(); ++i) x[i] = *reinterpret_cast<const v4i *>(xrow[i] + 32 * xb + 16 * (c & 1));
}

// Whole stages (the row-scale formats and group scales): a stream is a base that is the
// same for the whole wave (the expert's matrix from the wave's row tile, or
// the activations) plus the lane's 32-bit byte offset, and a stage moves the
// base only, so the loads take scalar bases and one vector offset each and a
// stage costs no vector address arithmetic. The bytes are load_w's and
// load_x's without their clamps, which whole stages never need.
template <int WB>
__device__ __forceinline__ uint32_t w_lane_off(long rowb)
{
    const int lane = threadIdx.x & 63, c = lane & 7;
    const long o = (long)(lane >> 3) * rowb + (WB == 8 ? (c >> 2) * (rowb / 2) + 16 * (c & 3) : (WB == 4 ? 16 : 8) * c);
    return (uint32_t)o;
}

template <int WB>
__device__ __forceinline__ void load_w_u(typename WReg<WB>::type (&w)[4], int s, const uint8_t *base, uint32_t off,
                                         long rowb)
{
    typedef typename WReg<WB>::type R;
    constexpr long SB = (WB == 2 ? 8 : 16) * stage_blocks<WB>();   // bytes of a row (int8: of a half) per stage
    const uint8_t *sb = base + SB * s;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = *reinterpret_cast<const R *>(sb + (long)(8 * j) * rowb + off);
}

template <int WB>
__device__ __forceinline__ void load_x_u(v4i (&x)[x_loads<WB>()], int s, const int8_t *act,
                                         const uint32_t (&off)[x_loads<WB>()])
{
    const int8_t *sb = act + (long)(32 * stage_blocks<WB>()) * s;
#pragma unroll
    for (int i = 0; i < x_loads<WB>(); ++i) x[i] = *reinterpret_cast<const v4i *>(sb + off[i]);
}

// Wave 0 loads the tile's scales, 4 blocks per lane: int4, pair l/2 and
// blocks 4*(l&1).. of the stage; int8, pair l (lanes 0-31). A 16-byte load
// when 4 | nblk, clamped in bounds.
template <int WB>
__device__ __forceinline__ v4f load_d(int s, int nblk, const float *drow, bool vec_scales)
{
    constexpr int KS = stage_blocks<WB>();
    const int b = s * KS + (KS == 8 ? 4 * (threadIdx.x & 1) : 0);
    if (vec_scales) return *reinterpret_cast<const v4f *>(drow + min(b, nblk - 4));
    v4f d;
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k] = drow[min(b + k, nblk - 1)];
    return d;
}

// Group scales of stage s for the wave's 32 rows: lane l takes row l % 32
// and slots 2*(l/32), 2*(l/32)+1, i.e. groups (s*KS >> gsh) + slot of that
// row (clamped in bounds; slots past the stage's groups are never read).
// srow: the lane's row of scales, ngs groups long.
typedef float v2f __attribute__((ext_vector_type(2)));

template <int WB>
__device__ __forceinline__ v2f load_s(int s, int gsh, const float *srow, int ngs)
{
    const int g = ((s * stage_blocks<WB>()) >> gsh) + 2 * ((threadIdx.x & 63) >> 5);
    return v2f{srow[min(g, ngs - 1)], srow[min(g + 1, ngs - 1)]};
}

template <int NM, int WB>
__device__ __forceinline__ void store_s(StageLds<NM, WB> &sm, int m, v2f sv)
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int k = 2 * (lane >> 5), r = lane & 31;
    sm.sg[wave][m][k][r] = (double)sv[0];
    sm.sg[wave][m][k + 1][r] = (double)sv[1];
}

// Lane l's piece (chunk l % 8) of row n of slot (wave, m).
template <int NM, int WB>
__device__ __forceinline__ void store_w_row(StageLds<NM, WB> &sm, int wave, int m, int n, typename WReg<WB>::type w)
{
    const int k = threadIdx.x & 7;
    if constexpr (WB == 2 || WB == WB_GROUPS) {   // 8-byte piece k: half k % 2 of chunk k / 2
        char *row = reinterpret_cast<char *>(&sm.w[wave][m][n][0]);
        *reinterpret_cast<v2i *>(row + 16 * ((k >> 1) ^ wsw<2>(n)) + 8 * (k & 1)) = w;
    } else {
        sm.w[wave][m][n][k ^ wsw<WB>(n)] = w;
    }
}

template <int NM, int WB>
__device__ __forceinline__ void store_w(StageLds<NM, WB> &sm, int m, const typename WReg<WB>::type (&w)[4])
{
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) store_w_row<NM, WB>(sm, wave, m, 8 * j + (lane >> 3), w[j]);
}

template <int NM, int WB>
__device__ __forceinline__ void store_x(StageLds<NM, WB> &sm, int buf, const v4i (&x)[x_loads<WB>()])
{
    constexpr int XC = stage_xc<WB>();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < x_loads<WB>(); ++i) {
        const int p = 8 * wave + (64 / XC) * i + lane / XC;
        sm.x[buf][p][(lane & (XC - 1)) ^ xsw<WB>(p)] = x[i];
    }
}

// Scales are staged as the f64 factors the rescale multiplies by: d_b/16
// for int4 (the nibble trick's x16 undone, exact), d_b/64 for int2 (its
// codes unpacked x64), d_b for int8, and 0 for
// pairs past the tile's np, so the MFMA loops do no conversions. Kept
// pair-minor: the lanes reading one block pair's factors read contiguous
// bytes.
template <int WB>
__device__ __forceinline__ int d_pair(int lane) { return stage_blocks<WB>() == 8 ? (lane >> 1) : lane; }

// Slot of pair p's factors in the pair-row form (below): the lane that reads
// them, (lane & 15) + 16 * (lane >> 5), so the 16 lanes of one LDS access
// read 16 different slots.
__device__ __forceinline__ int pr_slot(int p) { return (p & 3) + 4 * ((p >> 3) & 3) + 16 * ((p >> 2) & 1); }

template <int NM, int WB, bool PR = false>
__device__ __forceinline__ void store_d(StageLds<NM, WB> &sm, int buf, v4f d, int np)
{
    const int lane = threadIdx.x & 63;
    const int p = d_pair<WB>(lane), jp = stage_blocks<WB>() == 8 ? 2 * (lane & 1) : 0;
    if (p >= TILE_N) return;                     // int8: lanes 32-63 stage nothing
    const double v = p < np ? (int4_codes<WB>() ? 0.0625 : WB == 2 ? 0.015625 : 1.0) : 0.0;
    const int slot = PR ? pr_slot(p) : p;
    sm.d[buf][jp][slot] = v2d{(double)d[0] * v, (double)d[1] * v};
    sm.d[buf][jp + 1][slot] = v2d{(double)d[2] * v, (double)d[3] * v};
}

// Factors of blocks j and j+1 (j even) of the stage for pair n.
template <int NM, int WB>
__device__ __forceinline__ v2d read_d2(const StageLds<NM, WB> &sm, int buf, int n, int j)
{
    return sm.d[buf][j >> 1][n];
}

// Global row of this wave's share of the tile's activation loads (pair
// 8*wave + (64/XC)*i + lane/XC; pairs past np read the tile's first pair).
template <int WB>
__device__ __forceinline__ int stage_pair(int i, int np)
{
    constexpr int XC = stage_xc<WB>();
    const int p = 8 * (threadIdx.x >> 6) + (64 / XC) * i + (threadIdx.x & 63) / XC;
    return p < np ? p : 0;
}

// Narrow tiles. A tile holding at most 16 pairs (the last tile of an expert
// with n % 32 <= 16 pairs, which at prefill is most experts) runs
// v_mfma_i32_16x16x32_i8 twice per block instead of the 32x32 MFMA: rows
// 0-15 and 16-31 of the wave's 32 against the tile's 16 pairs. Lane l then
// holds pair l%16 and the 8 k of quarter q = l/16 of the block (8-group q:
// weight bytes 4q..4q+3, activation bytes 8q..8q+7 of the reordered block,
// the same k for both operands), and gets rows 4q..4q+3 of each MFMA's
// 16x16 result. Each lane rescales 8 elements per block instead of 16, so
// a narrow tile costs about half the vector work of a 32-pair one.
template <bool NARROW> struct TileShape;
template <> struct TileShape<false> { static constexpr int NACC = 16, NPAIR = 32; };
template <> struct TileShape<true> { static constexpr int NACC = 8, NPAIR = 16; };

// Row of accumulator i of this lane within the wave's 32 rows.
template <bool NARROW>
__device__ __forceinline__ int acc_row(int i, int lane)
{
    if constexpr (NARROW) return 16 * (i >> 2) + 4 * (lane >> 4) + (i & 3);
    else return tile_row(i, lane >> 5);
}

// Pair of this lane's accumulators within the tile.
template <bool NARROW>
__device__ __forceinline__ int acc_pair(int lane) { return NARROW ? (lane & 15) : (lane & 31); }

// Both unpacked nibble dwords of one packed dword (elements of one 8-group,
// x16, in the reordered order) as the 8-byte operand of the 16x16x32 MFMA.
__device__ __forceinline__ long unpack4(uint32_t w)
{
    const uint32_t m = 0xF0F0F0F0u;
    return (long)(((unsigned long long)(w & m) << 32) | (unsigned long long)((w << 4) & m));
}

// One int2 dword (16 columns) as the 16 operand bytes x64, in the
// reordered activation order: fields 0, 1, 2, 3 of its bytes are columns
// 2k, 2k+1, 2k+8, 2k+9, i.e. the activation dwords 0..3 of those columns.
__device__ __forceinline__ v4i unpack16_2b(uint32_t w)
{
    const uint32_t m = 0xC0C0C0C0u;
    return v4i{(int)((w << 6) & m), (int)((w << 4) & m), (int)((w << 2) & m), (int)(w & m)};
}

// The same for one 8-group: the first (hi = 0) or second 8 columns of the
// dword, as the 16x16x32 MFMA's 8-byte operand.
__device__ __forceinline__ long unpack8_2b(uint32_t w, int hi)
{
    const uint32_t m = 0xC0C0C0C0u;
    const uint32_t a = hi ? (w << 2) & m : (w << 6) & m;
    const uint32_t b = hi ? w & m : (w << 4) & m;
    return (long)(((unsigned long long)b << 32) | (unsigned long long)a);
}

// The 16 bytes of block j (of the stage) that lane half `half` multiplies,
// as the 32x32x32 MFMA's operand, for blocks j and j+1: int4 chunks hold a
// whole block (each half takes its 8 packed bytes of both, read directly or
// by one 16-byte read and a permlane swap, then the nibbles are unpacked
// x16); int8 chunks hold one half of a block.
template <int NM, int WB>
__device__ __forceinline__ void w_pair(const StageLds<NM, WB> &sm, int wave, int m, int n, int half, int sw, int j,
                                       v4i &a, v4i &b)
{
    if constexpr (int4_codes<WB>() && NM == 2) {
        // both matrices per wave: one 16-byte read and the swap (reading the
        // two 8-byte halves directly costs that kernel 4 spilled registers)
        const uint4 wp = as_u4(sm.w[wave][m][n][(j + half) ^ sw]);
        uint2 wa, wb;
        split_pair(wp, wa, wb);
        a = unpack8(wa);
        b = unpack8(wb);
    } else if constexpr (int4_codes<WB>()) {    // half h reads its 8 packed bytes of each block
        const char *row = reinterpret_cast<const char *>(&sm.w[wave][m][n][0]);
        a = unpack8(*reinterpret_cast<const uint2 *>(row + 16 * (j ^ sw) + 8 * half));
        b = unpack8(*reinterpret_cast<const uint2 *>(row + 16 * ((j + 1) ^ sw) + 8 * half));
    } else if constexpr (WB == 2) {              // blocks j, j+1 share chunk j/2; half h takes dword h of each
        const char *ch = reinterpret_cast<const char *>(&sm.w[wave][m][n][(j >> 1) ^ sw]);
        a = unpack16_2b(*reinterpret_cast<const uint32_t *>(ch + 4 * half));
        b = unpack16_2b(*reinterpret_cast<const uint32_t *>(ch + 8 + 4 * half));
    } else {
        a = sm.w[wave][m][n][(4 * half + j) ^ sw];
        b = sm.w[wave][m][n][(4 * half + j + 1) ^ sw];
    }
}

// The 8 bytes of 8-group q of block blk for row r, as the 16x16x32 MFMA's
// operand: int4, the packed dword of the group unpacked x16; int8, the
// group's bytes in the block's half q/2.
template <int NM, int WB>
__device__ __forceinline__ long w_group(const StageLds<NM, WB> &sm, int wave, int m, int r, int sw, int blk, int q)
{
    const char *row = reinterpret_cast<const char *>(&sm.w[wave][m][r][0]);
    if constexpr (int4_codes<WB>()) {
        return unpack4(*reinterpret_cast<const uint32_t *>(row + 16 * (blk ^ sw) + 4 * q));
    } else if constexpr (WB == 2) {              // dword q/2 of the block; its first or second 8 columns
        const uint32_t w = *reinterpret_cast<const uint32_t *>(row + 16 * ((blk >> 1) ^ sw) + 8 * (blk & 1) + 4 * (q >> 1));
        return unpack8_2b(w, q & 1);
    } else {
        return *reinterpret_cast<const long *>(row + 16 * ((4 * (q >> 1) + blk) ^ sw) + 8 * (q & 1));
    }
}

// Group scales: acc += s_g * (f * c), the oracle's term and order. f * c
// (the block factor times the int32 result) is exact in f64; the product
// with the group scale and the sum are rounded one at a time, so nothing
// here may become an FMA.
__device__ __forceinline__ double gs_term(double acc, int c, double f, double sg)
{
#pragma clang fp contract(off)
    const double p = (double)c * f;
    return acc + sg * p;
}

// One matrix over the stage's blocks, adding every block's int32 results
// times its f64 factor into acc (with group scales, each term times its
// row's group scale; gsh: log2(group / 32)). m: the matrix's LDS slot; buf: the stage's
// activation buffer; b0: its first block.
template <bool FULL, bool NARROW, int NM, int WB>
__device__ __forceinline__ void stage_pass(const StageLds<NM, WB> &sm, int m, double (&acc)[TileShape<NARROW>::NACC],
                                           int buf, int b0, int nblk, int gsh = 0)
{
    constexpr bool GS = WB == WB_GROUPS;
    const int g0 = b0 >> gsh;                    // the stage's first group
    constexpr int KS = stage_blocks<WB>();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if constexpr (!NARROW) {
        const v16i zero = {};
        const int n = lane & 31, half = lane >> 5;
        const int sw = wsw<WB>(n), sx = xsw<WB>(n);
        // Both MFMAs of a block pair are issued before either result is
        // rescaled: the second runs on the matrix core while the vector
        // unit converts and accumulates the first.
#pragma unroll
        for (int j = 0; j < KS; j += 2) {
            if (!FULL && b0 + j >= nblk) break;          // uniform: the stage's valid blocks
            const bool two = FULL || b0 + j + 1 < nblk;
            v4i ua, ub;
            w_pair<NM, WB>(sm, wave, m, n, half, sw, j, ua, ub);
            const int4 x0 = as_i4(sm.x[buf][n][(2 * j + half) ^ sx]);
            const int4 x1 = as_i4(sm.x[buf][n][(2 * j + 2 + half) ^ sx]);
            const v2d dd = read_d2<NM, WB>(sm, buf, n, j);
            const v16i ca = __builtin_amdgcn_mfma_i32_32x32x32_i8(ua, v4i{x0.x, x0.y, x0.z, x0.w}, zero, 0, 0, 0);
            const v16i cb = two ? __builtin_amdgcn_mfma_i32_32x32x32_i8(ub, v4i{x1.x, x1.y, x1.z, x1.w}, zero, 0, 0, 0)
                                : zero;
            if constexpr (GS) {
                const double *sa = sm.sg[wave][m][((b0 + j) >> gsh) - g0];
                const double *sb = sm.sg[wave][m][((b0 + j + 1) >> gsh) - g0];
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = gs_term(acc[i], ca[i], dd[0], sa[tile_row(i, half)]);
                if (two) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[i] = gs_term(acc[i], cb[i], dd[1], sb[tile_row(i, half)]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = fma((double)ca[i], dd[0], acc[i]);
                if (two) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[i] = fma((double)cb[i], dd[1], acc[i]);
                }
            }
        }
    } else {
        const v4i zero = {};
        const int pr = lane & 15, q = lane >> 4;
        const int sx = xsw<WB>(pr);
        const int r0 = pr, r1 = pr + 16;                 // the lane's weight rows of the two MFMAs
        const int sw0 = wsw<WB>(r0), sw1 = wsw<WB>(r1);
        // the four MFMAs of a block pair are issued before any result is
        // rescaled (see the 32-pair form)
#pragma unroll
        for (int j = 0; j < KS; j += 2) {
            if (!FULL && b0 + j >= nblk) break;
            const bool two = FULL || b0 + j + 1 < nblk;
            const v2d dd = read_d2<NM, WB>(sm, buf, pr, j);
            v4i c[2][2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int blk = j + jj;
                if (jj == 1 && !two) {
                    c[1][0] = zero;
                    c[1][1] = zero;
                    break;
                }
                const char *xr = reinterpret_cast<const char *>(&sm.x[buf][pr][(2 * blk + (q >> 1)) ^ sx]);
                const long B = *reinterpret_cast<const long *>(xr + 8 * (q & 1));
                c[jj][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(w_group<NM, WB>(sm, wave, m, r0, sw0, blk, q), B, zero, 0, 0, 0);
                c[jj][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(w_group<NM, WB>(sm, wave, m, r1, sw1, blk, q), B, zero, 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                if (jj == 1 && !two) break;
                if constexpr (GS) {
                    const double *sr = sm.sg[wave][m][((b0 + j + jj) >> gsh) - g0];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[i] = gs_term(acc[i], c[jj][0][i], dd[jj], sr[4 * q + i]);
                        acc[4 + i] = gs_term(acc[4 + i], c[jj][1][i], dd[jj], sr[16 + 4 * q + i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[i] = fma((double)c[jj][0][i], dd[jj], acc[i]);
                        acc[4 + i] = fma((double)c[jj][1][i], dd[jj], acc[4 + i]);
                    }
                }
            }
        }
    }
}

// Pair-row form (row-scale formats, whole stages). The tile's pairs are the
// MFMA's A rows and the weight rows its B columns, so lane l holds weight
// row l%32 and, in accumulator i, pair 8*(i/4) + 4*(l/32) + i%4: the four
// accumulators of group g hold pairs 8g..8g+7 in every lane, and a tile of
// np pairs keeps and rescales only its first G = ceil(np/8) groups, where
// the pair-column form pays for 32 (or, at most 16 pairs, 16) pair slots.
// The factor of accumulator i belongs to one pair per 16-lane row; lane
// (i, row) reads that pair's factors from LDS and v_fmac_f64 takes them
// with DPP row_newbcast:i, so the rescale stays one conversion and one f64
// FMA per element and block, with the same rounding as the other form.
//
// Four accumulators of group I0/4: acc += f(lane I0+k of the row) * c, one
// fused multiply-add each. The s_nop gives the two wait states a DPP
// operand needs after a vector write of its register.
template <int I0>
__device__ __forceinline__ void fmac4_bcast(double &a0, double &a1, double &a2, double &a3, double f, double c0,
                                            double c1, double c2, double c3)
{
    asm("s_nop 1\n\t"
        "v_fmac_f64_dpp %0, %4, %5 row_newbcast:%9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f64_dpp %1, %4, %6 row_newbcast:%10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f64_dpp %2, %4, %7 row_newbcast:%11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f64_dpp %3, %4, %8 row_newbcast:%12 row_mask:0xf bank_mask:0xf"
        : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)
        : "v"(f), "v"(c0), "v"(c1), "v"(c2), "v"(c3), "i"(I0), "i"(I0 + 1), "i"(I0 + 2), "i"(I0 + 3));
}

// The conversions of a group stay next to its FMAs (vector instructions may
// not cross the barriers; memory and MFMA instructions may): converted
// ahead, a whole result would hold 32 more registers.
constexpr int PR_CROSS = 0x3FC;

template <int G>
__device__ __forceinline__ void rescale_pr(double (&acc)[4 * G], const v16i &c, double f)
{
    fmac4_bcast<0>(acc[0], acc[1], acc[2], acc[3], f, (double)c[0], (double)c[1], (double)c[2], (double)c[3]);
    __builtin_amdgcn_sched_barrier(PR_CROSS);
    if constexpr (G > 1) {
        fmac4_bcast<4>(acc[4], acc[5], acc[6], acc[7], f, (double)c[4], (double)c[5], (double)c[6], (double)c[7]);
        __builtin_amdgcn_sched_barrier(PR_CROSS);
    }
    if constexpr (G > 2) {
        fmac4_bcast<8>(acc[8], acc[9], acc[10], acc[11], f, (double)c[8], (double)c[9], (double)c[10], (double)c[11]);
        __builtin_amdgcn_sched_barrier(PR_CROSS);
    }
    if constexpr (G > 3) {
        fmac4_bcast<12>(acc[12], acc[13], acc[14], acc[15], f, (double)c[12], (double)c[13], (double)c[14],
                        (double)c[15]);
        __builtin_amdgcn_sched_barrier(PR_CROSS);
    }
}

// The lane index, opaque to the compiler: the epilogue's store addresses
// derive from it, so they are not computed before the K loop and held in
// registers through it.
__device__ __forceinline__ int after_loop(int lane)
{
    __asm__ volatile("" : "+v"(lane));
    return lane;
}

// Formats the pair-row form serves: one scale per weight row (with group
// scales each block term carries its own, which rounds apart from the FMA).
template <int WB> constexpr bool pr_form() { return WB == 4 || WB == 2 || WB == 8; }

// Pair of accumulator i of this lane in the pair-row form.
__device__ __forceinline__ int pr_pair(int i, int lane) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); }

// One matrix over a whole stage in the pair-row form (G groups); the wave's
// LDS slot holds one matrix (int4: the two 8-byte halves of each block).
template <int G, int WB>
__device__ __forceinline__ void stage_pass_pr(const StageLds<1, WB> &sm, double (&acc)[4 * G], int buf)
{
    constexpr int KS = stage_blocks<WB>();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int n = lane & 31, half = lane >> 5;
    const int sw = wsw<WB>(n), sx = xsw<WB>(n);
    const int fs = (lane & 15) + 16 * half;      // pr_slot of the pair whose factors this lane reads
    const v16i zero = {};
#pragma unroll
    for (int j = 0; j < KS; j += 2) {
        v4i ua, ub;
        w_pair<1, WB>(sm, wave, 0, n, half, sw, j, ua, ub);
        const v4i x0 = sm.x[buf][n][(2 * j + half) ^ sx];
        const v4i x1 = sm.x[buf][n][(2 * j + 2 + half) ^ sx];
        const v2d dd = sm.d[buf][j >> 1][fs];
        const v16i ca = __builtin_amdgcn_mfma_i32_32x32x32_i8(x0, ua, zero, 0, 0, 0);
        const v16i cb = __builtin_amdgcn_mfma_i32_32x32x32_i8(x1, ub, zero, 0, 0, 0);
        rescale_pr<G>(acc, ca, dd[0]);
        rescale_pr<G>(acc, cb, dd[1]);
    }
}

// FULL: the K blocks fill whole stages (nblk % KS == 0), so a stage's blocks
// need no bounds tests and the scheduler sees a stage as straight-line code.
//
// Two gate/up tile forms. Paired waves (gateup_tile_paired): wave w runs matrix
// w & 1 (0 gate, 1 up) of row tile rg * GU_RT + (w >> 1), so each wave holds
// one matrix's accumulators and the four waves still share one stage of
// activations; at the end the gate wave hands its g values to its up partner
// through LDS. Both matrices per wave (gateup_tile_both): four row tiles per
// workgroup, each wave running the gate pass, then the up pass of a stage.
constexpr int GU_RT = WAVES / 2;   // row tiles per gate/up workgroup of paired waves

template <bool FULL, bool NARROW, int WB, int PRG = 0>
__device__ __forceinline__ void gateup_tile_paired(const GroupedArgs &a, StageLds<1, WB> &sm, int e, int p0,
                                                   int np, int rt, int mat, bool rows_ok)
{
    static_assert(PRG == 0 || (FULL && pr_form<WB>()), "the pair-row form takes row scales in whole stages");
    constexpr int NACC = PRG ? 4 * PRG : TileShape<NARROW>::NACC, KS = stage_blocks<WB>(), NXL = x_loads<WB>();
    const int n_rt = a.I / QK;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nblk = a.H / QK;
    constexpr bool GS = WB == WB_GROUPS;
    const long rowb = (long)a.H * code_bits<WB>() / 8;
    const long wrow0 = (long)e * a.I + (long)min(rt, n_rt - 1) * QK + (lane >> 3);
    const uint8_t *wrow = (mat ? a.q_b : a.q_a) + wrow0 * rowb;
    const int ngs = nblk >> a.gsh;               // group scales per row
    const float *srow = (mat ? a.s_b : a.s_a) + ((long)e * a.I + (long)min(rt, n_rt - 1) * QK + (lane & 31)) * ngs;
    v2f sn = {};
    const int8_t *xrow[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i) xrow[i] = a.act + (long)a.pair_tok[p0 + stage_pair<WB>(i, np)] * a.H;
    // whole stages: scalar-based streams (rt, mat: the same in every lane of the wave)
    constexpr bool U = FULL && (pr_form<WB>() || WB == WB_GROUPS);
    const int rtu = __builtin_amdgcn_readfirstlane(min(rt, n_rt - 1)), matu = __builtin_amdgcn_readfirstlane(mat);
    const uint8_t *wbase = (matu ? a.q_b : a.q_a) + ((long)e * a.I + (long)rtu * QK) * rowb;
    const uint32_t woff = w_lane_off<WB>(rowb);
    uint32_t xoff[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i)
        xoff[i] = (uint32_t)a.pair_tok[p0 + stage_pair<WB>(i, np)] * (uint32_t)a.H + 16u * (threadIdx.x & (stage_xc<WB>() - 1));
    const int pd = min(d_pair<WB>(lane), TILE_N - 1) < np ? min(d_pair<WB>(lane), TILE_N - 1) : 0;
    const float *drow = a.act_s + (long)a.pair_tok[p0 + pd] * nblk;   // used by wave 0
    const bool vec_scales = nblk % 4 == 0;

    double acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = 0.0;

    // the next stage's rows and activations load while the current one
    // computes
    const int nst = (nblk + KS - 1) / KS;
    typename WReg<WB>::type wn[4];
    v4i xn[NXL];
    v4f dn = {};
    if constexpr (U) load_x_u<WB>(xn, 0, a.act, xoff);
    else load_x<WB>(xn, 0, nblk, xrow);
    if (wave == 0) dn = load_d<WB>(0, nblk, drow, vec_scales);
    if (rows_ok) {
        if constexpr (U) load_w_u<WB>(wn, 0, wbase, woff, rowb);
        else load_w<WB>(wn, 0, nblk, wrow, rowb);
        if constexpr (GS) sn = load_s<WB>(0, a.gsh, srow, ngs);
        store_w<1, WB>(sm, 0, wn);
        if constexpr (GS) store_s<1, WB>(sm, 0, sn);
    }
    store_x<1, WB>(sm, 0, xn);
    if (wave == 0) store_d<1, WB, PRG != 0>(sm, 0, dn, np);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const bool more = s + 1 < nst;
        if (more) {
            if constexpr (U) load_x_u<WB>(xn, s + 1, a.act, xoff);
            else load_x<WB>(xn, s + 1, nblk, xrow);
            if (wave == 0) dn = load_d<WB>(s + 1, nblk, drow, vec_scales);
            if (rows_ok) {
                if constexpr (U) load_w_u<WB>(wn, s + 1, wbase, woff, rowb);
                else load_w<WB>(wn, s + 1, nblk, wrow, rowb);
                if constexpr (GS) sn = load_s<WB>(s + 1, a.gsh, srow, ngs);
            }
        }
        issue_fence();
        if constexpr (PRG) {
            if (rows_ok) stage_pass_pr<PRG, WB>(sm, acc, s & 1);
        } else {
            if (rows_ok) stage_pass<FULL, NARROW, 1, WB>(sm, 0, acc, s & 1, s * KS, nblk, a.gsh);
        }
        issue_fence();
        if (more) {
            if (rows_ok) {
                store_w<1, WB>(sm, 0, wn);
                if constexpr (GS) store_s<1, WB>(sm, 0, sn);
            }
            store_x<1, WB>(sm, (s + 1) & 1, xn);
            if (wave == 0) store_d<1, WB, PRG != 0>(sm, (s + 1) & 1, dn, np);
        }
        __syncthreads();
    }
    // The weight stages are done with: the gate wave leaves g (f32, after
    // its row scale) in its own weight slot, [accumulator][lane], for the up
    // wave of the same row tile (the next wave), whose lanes hold the same
    // (row, pair) elements.
    float *xg = reinterpret_cast<float *>(&sm.w[wave & ~1][0][0][0]);
    if constexpr (PRG) {
        // pair-row form: one row (lane % 32) and so one row scale per lane.
        // Each wave leaves its g or u values (after the row scale, f32) in an
        // LDS area of its own, 16 x 64 floats: its weight slot, or with int2
        // (whose weight slot is a quarter of that) a quarter of the
        // activation buffers, free after the last stage's barrier. One copy
        // of the SwiGLU and Q8 code (a loop, not unrolled) then serves every
        // accumulator; each accumulator's pair spans the 32 lanes of a half,
        // which take its Q8 block together.
        constexpr bool IN_X = sizeof(sm.w[0]) < 16 * 64 * sizeof(float);
        static_assert(!IN_X || sizeof(sm.x) >= WAVES * 16 * 64 * sizeof(float), "g and u fit the activation buffers");
        auto area = [&](int wv) -> float * {
            return IN_X ? reinterpret_cast<float *>(&sm.x[0][0][0]) + wv * 16 * 64
                        : reinterpret_cast<float *>(&sm.w[wv][0][0][0]);
        };
        const int ln = after_loop(lane), r = ln & 31;
        const long grow = (long)e * a.I + (long)rt * QK + r;
        if (rows_ok) {
            const double sc = (double)(mat ? a.s_b : a.s_a)[grow];
            float *own = area(wave);
#pragma unroll
            for (int i = 0; i < NACC; ++i) own[i * 64 + ln] = (float)(sc * acc[i]);
        }
        __syncthreads();
        if (!rows_ok || mat == 0) return;
        xg = area(wave & ~1);
        const float *xu = area(wave);
#pragma unroll 1
        for (int i = 0; i < NACC; ++i) {
            const float gf = xg[i * 64 + ln], uf = xu[i * 64 + ln];
            const float hv = (float)(silu_f64((double)gf) * (double)uf);
            float amax = fmaxf(0.0f, fabsf(hv));
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
            const int pn = pr_pair(i, ln);
            if (pn < np) {
                float d, id;
                q8_scale(amax, d, id);
                const long base = (long)(p0 + pn) * a.I + (long)rt * QK;
                a.h[base + r] = hv;
                a.hq[base + (r & ~7) + perm8(r & 7)] = (int8_t)round_clamp(__fmul_rn(hv, id), -127.0f, 127.0f);
                if (r == 0) a.hs[(long)(p0 + pn) * n_rt + rt] = d;
            }
        }
        return;
    }
    if (rows_ok && mat == 0) {
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            const long grow = (long)e * a.I + (long)rt * QK + acc_row<NARROW>(i, lane);
            // with group scales every block term carries its scale: no row scale
            xg[i * 64 + lane] = GS ? (float)acc[i] : (float)((double)a.s_a[grow] * acc[i]);
        }
    }
    __syncthreads();
    if (!rows_ok || mat == 0) return;
    // epilogue (up wave): h = silu(g)*u, Q8 over the tile's 32 rows per pair
    // (held by 2 lanes of a 32-pair tile, 4 lanes of a narrow one)
    float hv[NACC];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
        const long grow = (long)e * a.I + (long)rt * QK + acc_row<NARROW>(i, lane);
        const float gf = xg[i * 64 + lane];
        const float uf = GS ? (float)acc[i] : (float)((double)a.s_b[grow] * acc[i]);
        hv[i] = (float)(silu_f64((double)gf) * (double)uf);
        amax = fmaxf(amax, fabsf(hv[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if constexpr (NARROW) amax = fmaxf(amax, __shfl_xor(amax, 16));
    const int n = acc_pair<NARROW>(lane);
    if (n >= np) return;
    float d, id;
    q8_scale(amax, d, id);
    const long base = (long)(p0 + n) * a.I + (long)rt * QK;
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
        const int r = acc_row<NARROW>(i, lane);
        a.h[base + r] = hv[i];
        a.hq[base + (r & ~7) + perm8(r & 7)] = (int8_t)round_clamp(__fmul_rn(hv[i], id), -127.0f, 127.0f);
    }
    if (lane < TileShape<NARROW>::NPAIR) a.hs[(long)(p0 + n) * n_rt + rt] = d;
}

// Per stage: gate pass, then up pass, each wave holding both matrices of its
// row tile.
template <bool FULL, bool NARROW, int WB>
__device__ __forceinline__ void gateup_tile_both(const GroupedArgs &a, StageLds<2, WB> &sm, int e, int p0,
                                                 int np, int rt, bool rows_ok)
{
    constexpr int NACC = TileShape<NARROW>::NACC, KS = stage_blocks<WB>(), NXL = x_loads<WB>();
    const int n_rt = a.I / QK;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nblk = a.H / QK;
    constexpr bool GS = WB == WB_GROUPS;
    const long rowb = (long)a.H * code_bits<WB>() / 8;
    const long wrow0 = (long)e * a.I + (long)min(rt, n_rt - 1) * QK + (lane >> 3);
    const uint8_t *const wrow[2] = {a.q_a + wrow0 * rowb, a.q_b + wrow0 * rowb};
    const int ngs = nblk >> a.gsh;               // group scales per row
    const long srow0 = ((long)e * a.I + (long)min(rt, n_rt - 1) * QK + (lane & 31)) * ngs;
    const float *const srow[2] = {a.s_a + srow0, a.s_b + srow0};
    v2f sn = {};
    const int8_t *xrow[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i) xrow[i] = a.act + (long)a.pair_tok[p0 + stage_pair<WB>(i, np)] * a.H;
    const int pd = min(d_pair<WB>(lane), TILE_N - 1) < np ? min(d_pair<WB>(lane), TILE_N - 1) : 0;
    const float *drow = a.act_s + (long)a.pair_tok[p0 + pd] * nblk;   // used by wave 0
    const bool vec_scales = nblk % 4 == 0;

    double acc_g[NACC], acc_u[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) { acc_g[i] = 0.0; acc_u[i] = 0.0; }

    // Per stage: gate pass, then up pass. The next stage's gate rows and
    // activations load during the gate pass, its up rows during the up pass,
    // so only one matrix's stage is ever held in registers.
    const int nst = (nblk + KS - 1) / KS;
    typename WReg<WB>::type wn[4];
    v4i xn[NXL];
    v4f dn = {};
    load_x<WB>(xn, 0, nblk, xrow);
    if (wave == 0) dn = load_d<WB>(0, nblk, drow, vec_scales);
    if (rows_ok) {
        load_w<WB>(wn, 0, nblk, wrow[0], rowb);
        if constexpr (GS) sn = load_s<WB>(0, a.gsh, srow[0], ngs);
        store_w<2, WB>(sm, 0, wn);
        if constexpr (GS) store_s<2, WB>(sm, 0, sn);
        load_w<WB>(wn, 0, nblk, wrow[1], rowb);
        if constexpr (GS) sn = load_s<WB>(0, a.gsh, srow[1], ngs);
        store_w<2, WB>(sm, 1, wn);
        if constexpr (GS) store_s<2, WB>(sm, 1, sn);
    }
    store_x<2, WB>(sm, 0, xn);
    if (wave == 0) store_d<2, WB>(sm, 0, dn, np);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const bool more = s + 1 < nst;
        const int buf = s & 1, b0 = s * KS;
        if (more) {
            load_x<WB>(xn, s + 1, nblk, xrow);
            if (wave == 0) dn = load_d<WB>(s + 1, nblk, drow, vec_scales);
            if (rows_ok) {
                load_w<WB>(wn, s + 1, nblk, wrow[0], rowb);
                if constexpr (GS) sn = load_s<WB>(s + 1, a.gsh, srow[0], ngs);
            }
        }
        issue_fence();
        if (rows_ok) stage_pass<FULL, NARROW, 2, WB>(sm, 0, acc_g, buf, b0, nblk, a.gsh);
        issue_fence();
        if (more && rows_ok) {
            store_w<2, WB>(sm, 0, wn);
            if constexpr (GS) store_s<2, WB>(sm, 0, sn);
            load_w<WB>(wn, s + 1, nblk, wrow[1], rowb);
            if constexpr (GS) sn = load_s<WB>(s + 1, a.gsh, srow[1], ngs);
        }
        issue_fence();
        if (rows_ok) stage_pass<FULL, NARROW, 2, WB>(sm, 1, acc_u, buf, b0, nblk, a.gsh);
        issue_fence();
        if (more) {
            if (rows_ok) {
                store_w<2, WB>(sm, 1, wn);
                if constexpr (GS) store_s<2, WB>(sm, 1, sn);
            }
            store_x<2, WB>(sm, (s + 1) & 1, xn);
            if (wave == 0) store_d<2, WB>(sm, (s + 1) & 1, dn, np);
        }
        __syncthreads();
    }
    if (!rows_ok) return;
    // epilogue: g, u, h = silu(g)*u, Q8 over the tile's 32 rows per pair
    // (held by 2 lanes of a 32-pair tile, 4 lanes of a narrow one)
    float hv[NACC];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
        const long grow = (long)e * a.I + (long)rt * QK + acc_row<NARROW>(i, lane);
        // with group scales every block term carries its scale: no row scale
        const float gf = GS ? (float)acc_g[i] : (float)((double)a.s_a[grow] * acc_g[i]);
        const float uf = GS ? (float)acc_u[i] : (float)((double)a.s_b[grow] * acc_u[i]);
        hv[i] = (float)(silu_f64((double)gf) * (double)uf);
        amax = fmaxf(amax, fabsf(hv[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if constexpr (NARROW) amax = fmaxf(amax, __shfl_xor(amax, 16));
    const int n = acc_pair<NARROW>(lane);
    if (n >= np) return;
    float d, id;
    q8_scale(amax, d, id);
    const long base = (long)(p0 + n) * a.I + (long)rt * QK;
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
        const int r = acc_row<NARROW>(i, lane);
        a.h[base + r] = hv[i];
        a.hq[base + (r & ~7) + perm8(r & 7)] = (int8_t)round_clamp(__fmul_rn(hv[i], id), -127.0f, 127.0f);
    }
    if (lane < TileShape<NARROW>::NPAIR) a.hs[(long)(p0 + n) * n_rt + rt] = d;
}

// The form per weight format, as measured at the GLM-5.2 prefill shape:
// int8 and group-scaled weights pair the waves (13-16% faster there); int4
// and int2 in whole stages pair the waves in the pair-row form (int4 as fast
// as, int2 4% faster than, both matrices per wave in the pair-column form,
// which in the pair-row form runs out of registers); int4 and int2 in
// part-filled stages keep both matrices per wave.
template <bool FULL, int WB> constexpr bool gu_paired() { return WB == 8 || WB == WB_GROUPS || (FULL && (WB == 4 || WB == 2)); }
template <bool FULL, int WB> constexpr int gu_row_tiles() { return gu_paired<FULL, WB>() ? GU_RT : WAVES; }

template <bool FULL, int WB> struct GuLds { typedef StageLds<gu_paired<FULL, WB>() ? 1 : 2, WB> type; };

template <bool FULL, int WB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) k_gateup_mfma(GroupedArgs a)
{
    __shared__ typename GuLds<FULL, WB>::type sm;
    constexpr int RTW = gu_row_tiles<FULL, WB>();
    const int n_rt = a.I / QK;
    const int nrg = (n_rt + RTW - 1) / RTW;
    int tile, rg;
    tile_rg_tm(blockIdx.x, nrg, a.ntiles_max, tile, rg);
    if (tile >= a.ctrl[CTRL_N_TILES_GU]) return;          // uniform over the workgroup
    const int wave = threadIdx.x >> 6;
    const int2 td = a.tiles[tile];
    const int e = td.x, p0 = td.y;
    const int np = min(TILE_N, a.expert_off[e + 1] - p0);
    if constexpr (gu_paired<FULL, WB>()) {
        const int rt = rg * GU_RT + (wave >> 1), mat = wave & 1;
        const bool rows_ok = rt < n_rt;                   // waves past the last row tile only stage activations
        if constexpr (FULL && pr_form<WB>()) {           // pair-row form, the tile's 8-pair groups
            const int ng = (np + 7) >> 3;
            if (ng == 1) gateup_tile_paired<FULL, false, WB, 1>(a, sm, e, p0, np, rt, mat, rows_ok);
            else if (ng == 2) gateup_tile_paired<FULL, false, WB, 2>(a, sm, e, p0, np, rt, mat, rows_ok);
            else if (ng == 3) gateup_tile_paired<FULL, false, WB, 3>(a, sm, e, p0, np, rt, mat, rows_ok);
            else gateup_tile_paired<FULL, false, WB, 4>(a, sm, e, p0, np, rt, mat, rows_ok);
        } else {
            if (np <= 16) gateup_tile_paired<FULL, true, WB>(a, sm, e, p0, np, rt, mat, rows_ok);
            else gateup_tile_paired<FULL, false, WB>(a, sm, e, p0, np, rt, mat, rows_ok);
        }
    } else {
        const int rt = rg * WAVES + wave;
        const bool rows_ok = rt < n_rt;
        if (np <= 16) gateup_tile_both<FULL, true, WB>(a, sm, e, p0, np, rt, rows_ok);
        else gateup_tile_both<FULL, false, WB>(a, sm, e, p0, np, rt, rows_ok);
    }
}

template <bool FULL, bool NARROW, int WB, int PRG = 0>
__device__ __forceinline__ void down_tile(const GroupedArgs &a, StageLds<1, WB> &sm, int e, int p0, int np, int rt,
                                          bool rows_ok)
{
    static_assert(PRG == 0 || (FULL && pr_form<WB>()), "the pair-row form takes row scales in whole stages");
    constexpr int NACC = PRG ? 4 * PRG : TileShape<NARROW>::NACC, KS = stage_blocks<WB>(), NXL = x_loads<WB>();
    const int n_rt = a.H / QK;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nblk = a.I / QK;
    constexpr bool GS = WB == WB_GROUPS;
    const long rowb = (long)a.I * code_bits<WB>() / 8;
    const long wrow0 = (long)e * a.H + (long)min(rt, n_rt - 1) * QK + (lane >> 3);
    const uint8_t *wrow = a.q_a + wrow0 * rowb;
    const int ngs = nblk >> a.gsh;
    const float *srow = a.s_a + ((long)e * a.H + (long)min(rt, n_rt - 1) * QK + (lane & 31)) * ngs;
    v2f sn = {};
    const int8_t *xrow[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i) xrow[i] = a.act + (long)(p0 + stage_pair<WB>(i, np)) * a.I;
    // whole stages: scalar-based streams (rt: the same in every lane of the wave)
    constexpr bool U = FULL && (pr_form<WB>() || WB == WB_GROUPS);
    const int rtu = __builtin_amdgcn_readfirstlane(min(rt, n_rt - 1));
    const uint8_t *wbase = a.q_a + ((long)e * a.H + (long)rtu * QK) * rowb;
    const uint32_t woff = w_lane_off<WB>(rowb);
    uint32_t xoff[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i)
        xoff[i] = (uint32_t)(p0 + stage_pair<WB>(i, np)) * (uint32_t)a.I + 16u * (threadIdx.x & (stage_xc<WB>() - 1));
    const int pd = min(d_pair<WB>(lane), TILE_N - 1) < np ? min(d_pair<WB>(lane), TILE_N - 1) : 0;
    const float *drow = a.act_s + (long)(p0 + pd) * nblk;             // used by wave 0
    const bool vec_scales = nblk % 4 == 0;

    double acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = 0.0;

    const int nst = (nblk + KS - 1) / KS;
    typename WReg<WB>::type wn[4];
    v4i xn[NXL];
    v4f dn = {};
    if constexpr (U) load_x_u<WB>(xn, 0, a.act, xoff);
    else load_x<WB>(xn, 0, nblk, xrow);
    if (wave == 0) dn = load_d<WB>(0, nblk, drow, vec_scales);
    if (rows_ok) {
        if constexpr (U) load_w_u<WB>(wn, 0, wbase, woff, rowb);
        else load_w<WB>(wn, 0, nblk, wrow, rowb);
        if constexpr (GS) sn = load_s<WB>(0, a.gsh, srow, ngs);
        store_w<1, WB>(sm, 0, wn);
        if constexpr (GS) store_s<1, WB>(sm, 0, sn);
    }
    store_x<1, WB>(sm, 0, xn);
    if (wave == 0) store_d<1, WB, PRG != 0>(sm, 0, dn, np);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const bool more = s + 1 < nst;
        if (more) {
            if constexpr (U) load_x_u<WB>(xn, s + 1, a.act, xoff);
            else load_x<WB>(xn, s + 1, nblk, xrow);
            if (wave == 0) dn = load_d<WB>(s + 1, nblk, drow, vec_scales);
            if (rows_ok) {
                if constexpr (U) load_w_u<WB>(wn, s + 1, wbase, woff, rowb);
                else load_w<WB>(wn, s + 1, nblk, wrow, rowb);
                if constexpr (GS) sn = load_s<WB>(s + 1, a.gsh, srow, ngs);
            }
        }
        issue_fence();
        if constexpr (PRG) {
            if (rows_ok) stage_pass_pr<PRG, WB>(sm, acc, s & 1);
        } else {
            if (rows_ok) stage_pass<FULL, NARROW, 1, WB>(sm, 0, acc, s & 1, s * KS, nblk, a.gsh);
        }
        issue_fence();
        if (more) {
            if (rows_ok) {
                store_w<1, WB>(sm, 0, wn);
                if constexpr (GS) store_s<1, WB>(sm, 0, sn);
            }
            store_x<1, WB>(sm, (s + 1) & 1, xn);
            if (wave == 0) store_d<1, WB, PRG != 0>(sm, (s + 1) & 1, dn, np);
        }
        __syncthreads();
    }
    if constexpr (PRG) {                         // lane l: row l%32 of the tile, its pairs per accumulator
        if (!rows_ok) return;
        const int ln = after_loop(lane), r = ln & 31;
        const double rs = (double)a.s_a[(long)e * a.H + (long)rt * QK + r];
#pragma unroll
        for (int i = 0; i < NACC; ++i) {
            const int pn = pr_pair(i, ln);
            if (pn < np) a.ye[(long)(p0 + pn) * a.H + (long)rt * QK + r] = (float)(rs * acc[i]);
        }
        return;
    }
    const int n = acc_pair<NARROW>(lane);
    if (!rows_ok || n >= np) return;
    const long base = (long)(p0 + n) * a.H + (long)rt * QK;
    if constexpr (GS) {                          // every block term carries its group scale
#pragma unroll
        for (int i = 0; i < NACC; ++i) a.ye[base + acc_row<NARROW>(i, lane)] = (float)acc[i];
    } else {
        float rs[NACC];                          // row scales first: the stores below may not alias them
#pragma unroll
        for (int i = 0; i < NACC; ++i) rs[i] = a.s_a[(long)e * a.H + (long)rt * QK + acc_row<NARROW>(i, lane)];
#pragma unroll
        for (int i = 0; i < NACC; ++i) a.ye[base + acc_row<NARROW>(i, lane)] = (float)((double)rs[i] * acc[i]);
    }
}

template <bool FULL, int WB>
__global__ void __launch_bounds__(256) k_down_mfma(GroupedArgs a)
{
    __shared__ StageLds<1, WB> sm;
    const int n_rt = a.H / QK;
    const int nrg = (n_rt + WAVES - 1) / WAVES;
    int tile, rg;
    tile_rg_tm(blockIdx.x, nrg, a.ntiles_max, tile, rg);
    if (tile >= a.ctrl[CTRL_N_TILES_GU]) return;          // uniform over the workgroup
    const int wave = threadIdx.x >> 6;
    const int rt = rg * WAVES + wave;
    const bool rows_ok = rt < n_rt;
    const int2 td = a.tiles[tile];
    const int e = td.x, p0 = td.y;
    const int np = min(TILE_N, a.expert_off[e + 1] - p0);
    if constexpr (FULL && pr_form<WB>()) {               // pair-row form, the tile's 8-pair groups
        const int ng = (np + 7) >> 3;
        if (ng == 1) down_tile<FULL, false, WB, 1>(a, sm, e, p0, np, rt, rows_ok);
        else if (ng == 2) down_tile<FULL, false, WB, 2>(a, sm, e, p0, np, rt, rows_ok);
        else if (ng == 3) down_tile<FULL, false, WB, 3>(a, sm, e, p0, np, rt, rows_ok);
        else down_tile<FULL, false, WB, 4>(a, sm, e, p0, np, rt, rows_ok);
    } else {
        if (np <= 16) down_tile<FULL, true, WB>(a, sm, e, p0, np, rt, rows_ok);
        else down_tile<FULL, false, WB>(a, sm, e, p0, np, rt, rows_ok);
    }
}

// Quarter-tile form (down launches smaller than one resident round of
// workgroups, such as the dense MLP's few pair tiles, and row-scale
// formats): one 32-row tile per workgroup instead of four, so the launch has
// four times the workgroups and waves. Wave w takes rows 16 * (w & 1) and
// pairs 16 * (w >> 1) of the tile, 16 x 16, on v_mfma_i32_16x16x32_i8 (lane
// l: row and pair l % 16, the 8 k of quarter q = l / 16; result rows
// 4q..4q+3), so each lane rescales 4 elements per block: the same vector
// work per tile as the other forms, spread over four waves. The 32 rows are
// staged once for the workgroup, one chunk per thread, double-buffered in
// wave slots 0 and 1 (read by two waves each), beside the activations and
// factors as the other forms stage them, with two or four stages of loads
// in flight (a few registers here). Blocks are summed in block order.
template <bool FULL, int WB>
__device__ __forceinline__ void stage_pass_quad(const StageLds<1, WB> &sm, double (&acc)[4], int buf, int b0, int nblk)
{
    constexpr int KS = stage_blocks<WB>();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pr = lane & 15, q = lane >> 4;
    const int r = 16 * (wave & 1) + pr, p = 16 * (wave >> 1) + pr;   // A row, B pair of this lane
    const int sw = wsw<WB>(r), sx = xsw<WB>(p);
    const v4i zero = {};
#pragma unroll
    for (int j = 0; j < KS; j += 2) {
        if (!FULL && b0 + j >= nblk) break;
        const bool two = FULL || b0 + j + 1 < nblk;
        const v2d dd = read_d2<1, WB>(sm, buf, p, j);
        v4i c[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int blk = j + jj;
            if (jj == 1 && !two) {
                c[1] = zero;
                break;
            }
            const char *xr = reinterpret_cast<const char *>(&sm.x[buf][p][(2 * blk + (q >> 1)) ^ sx]);
            const long B = *reinterpret_cast<const long *>(xr + 8 * (q & 1));
            c[jj] = __builtin_amdgcn_mfma_i32_16x16x32_i8(w_group<1, WB>(sm, buf, 0, r, sw, blk, q), B, zero, 0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            if (jj == 1 && !two) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fma((double)c[jj][i], dd[jj], acc[i]);
        }
    }
}

template <bool FULL, int WB>
__device__ __forceinline__ void down_tile_quad(const GroupedArgs &a, StageLds<1, WB> &sm, int e, int p0, int np, int rt)
{
    constexpr int KS = stage_blocks<WB>(), NXL = x_loads<WB>();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, t = threadIdx.x;
    const int nblk = a.I / QK;
    const long rowb = (long)a.I * code_bits<WB>() / 8;
    const uint8_t *wrow = a.q_a + ((long)e * a.H + (long)rt * QK + (t >> 3)) * rowb;   // this thread's row
    const int8_t *xrow[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i) xrow[i] = a.act + (long)(p0 + stage_pair<WB>(i, np)) * a.I;
    const int pd = min(d_pair<WB>(lane), TILE_N - 1) < np ? min(d_pair<WB>(lane), TILE_N - 1) : 0;
    const float *drow = a.act_s + (long)(p0 + pd) * nblk;             // used by wave 0
    const bool vec_scales = nblk % 4 == 0;

    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    const int nst = (nblk + KS - 1) / KS;
    // QD stages of loads in flight: register set k holds stage s (s % QD ==
    // k) from its load until its store to LDS buffer s % 2, one iteration
    // before its compute; the loop runs QD stages per pass, so that every
    // register index is a constant. int8 stages are half as long as int4's
    // and hold fewer registers, so they keep twice as many in flight.
    constexpr int QD = WB == 8 ? 4 : 2;
    typename WReg<WB>::type wn[QD];
    v4i xn[QD][NXL];
    v4f dn[QD] = {};
    auto load = [&](int k, int st) {
        load_x<WB>(xn[k], st, nblk, xrow);
        if (wave == 0) dn[k] = load_d<WB>(st, nblk, drow, vec_scales);
        wn[k] = load_w_row<WB>(st, nblk, wrow, rowb);
    };
    auto store = [&](int k, int b) {             // buffer b was last read before the previous barrier
        store_w_row<1, WB>(sm, b, 0, t >> 3, wn[k]);
        store_x<1, WB>(sm, b, xn[k]);
        if (wave == 0) store_d<1, WB>(sm, b, dn[k], np);
    };
#pragma unroll
    for (int k = 0; k < QD; ++k)
        if (k < nst) load(k, k);
    store(0, 0);
    __syncthreads();
    for (int s0 = 0; s0 < nst; s0 += QD) {
#pragma unroll
        for (int k = 0; k < QD; ++k) {
            const int st = s0 + k;
            if (st >= nst) break;
            if (st + QD < nst) load(k, st + QD);     // set k: its stage st is in LDS already
            issue_fence();
            stage_pass_quad<FULL, WB>(sm, acc, k & 1, st * KS, nblk);
            issue_fence();
            if (st + 1 < nst) store((k + 1) % QD, (k + 1) & 1);
            __syncthreads();
        }
    }
    const int n = 16 * (wave >> 1) + (lane & 15);                     // this lane's pair
    if (n >= np) return;
    const int r0 = rt * QK + 16 * (wave & 1) + 4 * (lane >> 4);      // its first row
    float rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = a.s_a[(long)e * a.H + r0 + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) a.ye[(long)(p0 + n) * a.H + r0 + i] = (float)((double)rs[i] * acc[i]);
}

template <bool FULL, int WB>
__global__ void __launch_bounds__(256) k_down_quad(GroupedArgs a)
{
    static_assert(pr_form<WB>(), "row scales only: group-scaled terms are formed apart");
    __shared__ StageLds<1, WB> sm;
    const int n_rt = a.H / QK;
    int tile, rt;
    tile_rg_tm(blockIdx.x, n_rt, a.ntiles_max, tile, rt);
    if (tile >= a.ctrl[CTRL_N_TILES_GU]) return;          // uniform over the workgroup
    const int2 td = a.tiles[tile];
    const int e = td.x, p0 = td.y;
    const int np = min(TILE_N, a.expert_off[e + 1] - p0);
    down_tile_quad<FULL, WB>(a, sm, e, p0, np, rt);
}

// Quarter-tile gate/up (launches smaller than one resident round of
// workgroups, row-scale formats): one 32-row tile per workgroup, wave w
// running matrix w & 1 (gate, up) for pairs 16 * (w >> 1) .. + 15 of the
// tile, as the 16-pair form runs a narrow tile (two v_mfma_i32_16x16x32_i8
// per block, rows 0-15 and 16-31; lane l: pair l % 16, rows 4q..4q+3 of
// each, q = l / 16). Both matrices' 32 rows are staged once for the
// workgroup (two pieces per thread), double-buffered in wave slots 0 and 1;
// the gate waves leave g in slots 2 and 3 for the up waves, which take
// SwiGLU and Q8(h) as the paired waves do.
template <bool FULL, int WB>
__device__ __forceinline__ void stage_pass_gq(const StageLds<2, WB> &sm, double (&acc)[8], int buf, int b0, int nblk,
                                              int mat, int ph)
{
    constexpr int KS = stage_blocks<WB>();
    const int lane = threadIdx.x & 63;
    const int pr = lane & 15, q = lane >> 4, p = ph + pr;
    const int r0 = pr, r1 = pr + 16;
    const int sw0 = wsw<WB>(r0), sw1 = wsw<WB>(r1), sx = xsw<WB>(p);
    const v4i zero = {};
#pragma unroll
    for (int j = 0; j < KS; j += 2) {
        if (!FULL && b0 + j >= nblk) break;
        const bool two = FULL || b0 + j + 1 < nblk;
        const v2d dd = read_d2<2, WB>(sm, buf, p, j);
        v4i c[2][2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int blk = j + jj;
            if (jj == 1 && !two) {
                c[1][0] = zero;
                c[1][1] = zero;
                break;
            }
            const char *xr = reinterpret_cast<const char *>(&sm.x[buf][p][(2 * blk + (q >> 1)) ^ sx]);
            const long B = *reinterpret_cast<const long *>(xr + 8 * (q & 1));
            c[jj][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(w_group<2, WB>(sm, buf, mat, r0, sw0, blk, q), B, zero, 0, 0, 0);
            c[jj][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(w_group<2, WB>(sm, buf, mat, r1, sw1, blk, q), B, zero, 0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            if (jj == 1 && !two) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[i] = fma((double)c[jj][0][i], dd[jj], acc[i]);
                acc[4 + i] = fma((double)c[jj][1][i], dd[jj], acc[4 + i]);
            }
        }
    }
}

template <bool FULL, int WB>
__device__ __forceinline__ void gateup_tile_gq(const GroupedArgs &a, StageLds<2, WB> &sm, int e, int p0, int np, int rt)
{
    constexpr int KS = stage_blocks<WB>(), NXL = x_loads<WB>();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, t = threadIdx.x;
    const int mat = wave & 1, ph = 16 * (wave >> 1);
    const int n_rt = a.I / QK;
    const int nblk = a.H / QK;
    const long rowb = (long)a.H * code_bits<WB>() / 8;
    const long wr = ((long)e * a.I + (long)rt * QK + (t >> 3)) * rowb;    // this thread's row of both matrices
    const uint8_t *wg = a.q_a + wr, *wu = a.q_b + wr;
    const int8_t *xrow[NXL];
#pragma unroll
    for (int i = 0; i < NXL; ++i) xrow[i] = a.act + (long)a.pair_tok[p0 + stage_pair<WB>(i, np)] * a.H;
    const int pd = min(d_pair<WB>(lane), TILE_N - 1) < np ? min(d_pair<WB>(lane), TILE_N - 1) : 0;
    const float *drow = a.act_s + (long)a.pair_tok[p0 + pd] * nblk;   // used by wave 0
    const bool vec_scales = nblk % 4 == 0;

    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;
    const int nst = (nblk + KS - 1) / KS;
    typename WReg<WB>::type wn[2];
    v4i xn[NXL];
    v4f dn = {};
    auto load = [&](int st) {
        load_x<WB>(xn, st, nblk, xrow);
        if (wave == 0) dn = load_d<WB>(st, nblk, drow, vec_scales);
        wn[0] = load_w_row<WB>(st, nblk, wg, rowb);
        wn[1] = load_w_row<WB>(st, nblk, wu, rowb);
    };
    auto store = [&](int b) {                    // buffer b was last read before the previous barrier
        store_w_row<2, WB>(sm, b, 0, t >> 3, wn[0]);
        store_w_row<2, WB>(sm, b, 1, t >> 3, wn[1]);
        store_x<2, WB>(sm, b, xn);
        if (wave == 0) store_d<2, WB>(sm, b, dn, np);
    };
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const bool more = s + 1 < nst;
        if (more) load(s + 1);
        issue_fence();
        stage_pass_gq<FULL, WB>(sm, acc, s & 1, s * KS, nblk, mat, ph);
        issue_fence();
        if (more) store((s + 1) & 1);
        __syncthreads();
    }
    // the gate waves leave g (f32, after the row scale) in slot 2 + pair half,
    // [accumulator][lane]; the up wave of the same pairs reads it
    float *xg = reinterpret_cast<float *>(&sm.w[2 + (wave >> 1)][0][0][0]);
    static_assert(sizeof(sm.w[0]) >= 8 * 64 * sizeof(float), "g fits a spare weight slot");
    const long rbase = (long)e * a.I + (long)rt * QK;
    if (mat == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) xg[i * 64 + lane] = (float)((double)a.s_a[rbase + acc_row<true>(i, lane)] * acc[i]);
    }
    __syncthreads();
    if (mat == 0) return;
    float hv[8];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float gf = xg[i * 64 + lane];
        const float uf = (float)((double)a.s_b[rbase + acc_row<true>(i, lane)] * acc[i]);
        hv[i] = (float)(silu_f64((double)gf) * (double)uf);
        amax = fmaxf(amax, fabsf(hv[i]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    const int n = ph + (lane & 15);
    if (n >= np) return;
    float d, id;
    q8_scale(amax, d, id);
    const long base = (long)(p0 + n) * a.I + (long)rt * QK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = acc_row<true>(i, lane);
        a.h[base + r] = hv[i];
        a.hq[base + (r & ~7) + perm8(r & 7)] = (int8_t)round_clamp(__fmul_rn(hv[i], id), -127.0f, 127.0f);
    }
    if ((lane >> 4) == 0) a.hs[(long)(p0 + n) * n_rt + rt] = d;
}

template <bool FULL, int WB>
__global__ void __launch_bounds__(256) k_gateup_quad(GroupedArgs a)
{
    static_assert(pr_form<WB>(), "row scales only");
    __shared__ StageLds<2, WB> sm;
    const int n_rt = a.I / QK;
    int tile, rt;
    tile_rg_tm(blockIdx.x, n_rt, a.ntiles_max, tile, rt);
    if (tile >= a.ctrl[CTRL_N_TILES_GU]) return;          // uniform over the workgroup
    const int2 td = a.tiles[tile];
    const int e = td.x, p0 = td.y;
    const int np = min(TILE_N, a.expert_off[e + 1] - p0);
    gateup_tile_gq<FULL, WB>(a, sm, e, p0, np, rt);
}

// The launched grid counts tile slots past the batch's tiles too (their
// workgroups exit at once), so a grid of exactly one resident round still
// leaves CUs without work.
template <int WB>
bool gateup_small(unsigned grid)
{
    return (int)grid <= resident_wg_256(k_gateup_mfma<true, WB>);
}

// The quarter-tile form for a down launch smaller than one resident round of
// the four-row-tile kernel (measured: the int8 dense 64-token chunk's down
// launch, 96 workgroups of four row tiles, took 91.8 us).
template <int WB>
bool down_small(unsigned grid)
{
    return (int)grid < resident_wg_256(k_down_mfma<true, WB>);
}

GroupedArgs make_args(const WsLayout &lay, char *ws, const coli_moe_layer &L)
{
    GroupedArgs a;
    a.H = L.H; a.I = L.I;
    a.gsh = group_shift(L);
    a.ctrl = reinterpret_cast<const int *>(ws + lay.ctrl);
    a.tiles = reinterpret_cast<const int2 *>(ws + lay.tiles);
    a.expert_off = reinterpret_cast<const int *>(ws + lay.expert_off);
    a.pair_tok = reinterpret_cast<const int *>(ws + lay.pair_tok);
    a.h = reinterpret_cast<float *>(ws + lay.h);
    a.hq = reinterpret_cast<int8_t *>(ws + lay.hq);
    a.hs = reinterpret_cast<float *>(ws + lay.hs);
    a.ye = reinterpret_cast<float *>(ws + lay.ye);
    return a;
}

int max_tiles(const WsLayout &lay, const coli_moe_layer &L)
{
    return (lay.n_pairs + TILE_N - 1) / TILE_N + L.E + 1;
}

template <int WB>
void launch_gateup_quad(const GroupedArgs &a, const coli_moe_layer &L, const WsLayout &lay, hipStream_t s)
{
    const dim3 grid((unsigned)(max_tiles(lay, L) * (L.I / QK)));
    if ((L.H / QK) % stage_blocks<WB>() == 0) COLI_LAUNCH((k_gateup_quad<true, WB>), grid, dim3(64 * WAVES), 0, s, a);
    else COLI_LAUNCH((k_gateup_quad<false, WB>), grid, dim3(64 * WAVES), 0, s, a);
}

template <int WB>
void launch_down_quad(const GroupedArgs &a, const coli_moe_layer &L, const WsLayout &lay, hipStream_t s)
{
    const dim3 grid((unsigned)(max_tiles(lay, L) * (L.H / QK)));
    if ((L.I / QK) % stage_blocks<WB>() == 0) COLI_LAUNCH((k_down_quad<true, WB>), grid, dim3(64 * WAVES), 0, s, a);
    else COLI_LAUNCH((k_down_quad<false, WB>), grid, dim3(64 * WAVES), 0, s, a);
}

} // namespace

hipError_t launch_gateup_grouped(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    (void)T;
    GroupedArgs a = make_args(lay, ws, L);
    a.ntiles_max = max_tiles(lay, L);
    a.q_a = L.gate_q; a.s_a = L.gate_s; a.q_b = L.up_q; a.s_b = L.up_s;
    a.act = reinterpret_cast<const int8_t *>(ws + lay.xq);
    a.act_s = reinterpret_cast<const float *>(ws + lay.xs);
    const int nblk = L.H / QK;
    const bool pr_full = !L.group_size && (L.weight_bits == 4 || L.weight_bits == 2) && nblk % stage_blocks<4>() == 0;
    const int rtw = (L.group_size || L.weight_bits == 8 || pr_full) ? GU_RT : WAVES;   // gu_row_tiles<FULL, WB>()
    const int nrg = (L.I / QK + rtw - 1) / rtw;
    const dim3 grid((unsigned)(max_tiles(lay, L) * nrg));
    a.gsh = group_shift(L);
    // a grid smaller than one resident round takes the quarter-tile form (row scales)
    if (!L.group_size) {
        if (L.weight_bits == 8 && gateup_small<8>(grid.x)) { launch_gateup_quad<8>(a, L, lay, s); return hipGetLastError(); }
        if (L.weight_bits == 2 && gateup_small<2>(grid.x)) { launch_gateup_quad<2>(a, L, lay, s); return hipGetLastError(); }
        if (L.weight_bits == 4 && gateup_small<4>(grid.x)) { launch_gateup_quad<4>(a, L, lay, s); return hipGetLastError(); }
    }
    if (L.group_size) {
        if (nblk % stage_blocks<WB_GROUPS>() == 0)
            COLI_LAUNCH((k_gateup_mfma<true, WB_GROUPS>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_gateup_mfma<false, WB_GROUPS>), grid, dim3(64 * WAVES), 0, s, a);
    } else if (L.weight_bits == 8) {
        if (nblk % stage_blocks<8>() == 0) COLI_LAUNCH((k_gateup_mfma<true, 8>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_gateup_mfma<false, 8>), grid, dim3(64 * WAVES), 0, s, a);
    } else if (L.weight_bits == 2) {
        if (nblk % stage_blocks<2>() == 0) COLI_LAUNCH((k_gateup_mfma<true, 2>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_gateup_mfma<false, 2>), grid, dim3(64 * WAVES), 0, s, a);
    } else {
        if (nblk % stage_blocks<4>() == 0) COLI_LAUNCH((k_gateup_mfma<true, 4>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_gateup_mfma<false, 4>), grid, dim3(64 * WAVES), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_down_grouped(const coli_moe_layer &L, int T, const WsLayout &lay, char *ws, hipStream_t s)
{
    (void)T;
    GroupedArgs a = make_args(lay, ws, L);
    a.ntiles_max = max_tiles(lay, L);
    a.q_a = L.down_q; a.s_a = L.down_s; a.q_b = nullptr; a.s_b = nullptr;
    a.act = reinterpret_cast<const int8_t *>(ws + lay.hq);
    a.act_s = reinterpret_cast<const float *>(ws + lay.hs);
    const int nrg = (L.H / QK + WAVES - 1) / WAVES;
    const dim3 grid((unsigned)(max_tiles(lay, L) * nrg));
    a.gsh = group_shift(L);
    // whole stages (I/32 a multiple of the stage's blocks, as at I = 2048)
    // drop the per-block bounds tests; the row-scale formats then take the
    // pair-row form. A grid smaller than one resident round takes the
    // quarter-tile form (row scales).
    const int nblk = L.I / QK;
    if (!L.group_size) {
        if (L.weight_bits == 8 && down_small<8>(grid.x)) { launch_down_quad<8>(a, L, lay, s); return hipGetLastError(); }
        if (L.weight_bits == 2 && down_small<2>(grid.x)) { launch_down_quad<2>(a, L, lay, s); return hipGetLastError(); }
        if (L.weight_bits == 4 && down_small<4>(grid.x)) { launch_down_quad<4>(a, L, lay, s); return hipGetLastError(); }
    }
    if (L.group_size) {
        if (nblk % stage_blocks<WB_GROUPS>() == 0) COLI_LAUNCH((k_down_mfma<true, WB_GROUPS>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_down_mfma<false, WB_GROUPS>), grid, dim3(64 * WAVES), 0, s, a);
    } else if (L.weight_bits == 8) {
        if (nblk % stage_blocks<8>() == 0) COLI_LAUNCH((k_down_mfma<true, 8>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_down_mfma<false, 8>), grid, dim3(64 * WAVES), 0, s, a);
    } else if (L.weight_bits == 2) {
        if (nblk % stage_blocks<2>() == 0) COLI_LAUNCH((k_down_mfma<true, 2>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_down_mfma<false, 2>), grid, dim3(64 * WAVES), 0, s, a);
    } else {
        if (nblk % stage_blocks<4>() == 0) COLI_LAUNCH((k_down_mfma<true, 4>), grid, dim3(64 * WAVES), 0, s, a);
        else COLI_LAUNCH((k_down_mfma<false, 4>), grid, dim3(64 * WAVES), 0, s, a);
    }
    return hipGetLastError();
}

} // namespace coli
