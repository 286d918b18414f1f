// Eq. (1) of Nemotron-TwoTower (arXiv 2606.26493, section 2.1, "Bidirectional
// attention") for bf16 inputs on gfx950: the S queries of the noisy block
// attend to the concatenation of the layer-aligned context prefix (paged KV
// cache) and the block's own keys, with no mask.
//
// Shape of the computation. Query head h reads kv head g = h / G, so the S*G
// query rows (s, h in group g) of a sequence share every key: they form a
// dense 256-row tile and both products are MFMA contractions
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   S^T[key][row] = K[key][:] . Q[row][:]      (A = K tile from LDS, B = Q in registers)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row] (A = V tile read transposed from LDS,
//                                                B = P in registers)
// Computing the transposed score tile puts each lane's scores of one query
// row in the register layout the second product takes as its B operand, so P
// never leaves registers. The softmax is online (running max and sum per
// row) in the exp2 domain with the scale folded into one FMA; the running max
// is only moved when a tile's max exceeds it by more than 2^8, so the output
// accumulators are rarely rescaled.
//
// Work split. The prefix of each (sequence, kv head, row block) "pair" is cut
// into 64-key tiles, followed by one tile holding the S block keys. All
// tiles of all pairs are laid end to end and cut into segments of equal cost
// (tiles, plus a fixed charge for every piece start), one per workgroup, so
// every CU does the same work whatever the spread of prefix lengths. A pair that lies inside one segment is written
// directly; a pair cut by segment boundaries leaves one partial (O
// normalised, in the output's precision, and its fp32 LSE) per segment, merged by a second kernel. Segments are
// numbered so that consecutive ones run on the same XCD, which keeps a pair's
// partials in one L2.
//
// Schedule inside a workgroup. Eight waves own 32 query rows each; waves
// 0-3 bring the K half of every tile into LDS and waves 4-7 the V half, each
// wave 16 keys (one page id) per tile, with direct-to-LDS buffer loads: the
// data never passes through registers. K and V tiles are double-buffered in
// LDS: at the start of tile i's phase the K waves request K of tile i+1 and
// the V waves V of tile i (V is used one tile later), one phase before their
// first use. Per tile every wave runs one phase: the scores of tile i and,
// between those MFMAs, the softmax and PV product of tile i-1; then the mask
// and row max of tile i. Each wave waits for its own loads before the one
// workgroup barrier per tile that hands the buffers over. The query rows of
// the next piece are copied into LDS while the current one is computed.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;       // 32 query rows each; waves 0-3 load K, waves 4-7 load V
constexpr int kThreads = 64 * kWaves;
constexpr int kFinRows = 16;   // rows per merge workgroup (16 threads per row), 4 in the eight-group form
constexpr float kTau = 8.0f;  // lazy rescale threshold (log2 units)

constexpr float kLn2 = 0.693147180559945309f;
static_assert(kRows == 32 * kWaves, "one 32-row MFMA tile per wave");

template <int D>
struct Cfg {
    static constexpr int CPR = D / 8;           // 16-byte chunks per K/V row
    static constexpr int ROWB = D * 2;          // bytes of one K/V row
    static constexpr int TILEB = kTile * ROWB;  // LDS bytes of one K or V tile
    static constexpr int RPI = 64 / CPR;        // rows one 1 KB load instruction covers
    static constexpr int LPG = 16 / RPI;        // load instructions per wave and tile (16 keys)
    static constexpr int DS = D / 16;           // k-steps of the score product
    static constexpr int DT = D / 32;           // d tiles of the output product
    static constexpr int KSH = CPR == 16 ? 0 : 1;  // K swizzle: log2(rows per 256-byte bank period)
    static constexpr int G = CPR / 4;              // 64-byte groups per row
    static constexpr int VSH = G == 4 ? 0 : 1;     // V swizzle: log2(rows per bank period / 4 * G)
    static_assert((LPG == 2 || LPG == 4) && RPI * ROWB == 1024, "");
};

// LDS tiles keep the [key][d] layout in unpadded rows with XOR swizzles, so a
// direct-to-LDS load (each lane's 16 bytes land at 16 * lane) fills 1 KB of
// rows at once. A score-operand read (ds_read_b128) has 16 lanes read one
// 16-byte chunk c of 16 consecutive rows: chunk c of row r sits at position
// c ^ kswz(r), so the 16 lanes hit the 16 distinct 16-byte slots of a
// 256-byte bank period. A transposing V read (ds_read_b64_tr_b16) has 32 lanes
// read one 64-byte group of 4 consecutive rows: group g of row r sits at
// g ^ vswz(r), 4 distinct 64-byte slots. The loads put each lane's global
// chunk where the swizzle wants it.
template <int D>
__device__ __forceinline__ int kswz(int r) { return (r >> Cfg<D>::KSH) & (Cfg<D>::CPR - 1); }
template <int D>
__device__ __forceinline__ int vswz(int r) { return (r >> Cfg<D>::VSH) & (Cfg<D>::G - 1); }

// Element strides are 32-bit here (the host layer checks that they fit), which
// keeps the kernel's scalar state small.
struct Args {
    const uint16_t* Q;
    int qsb, qss, qsh;
    const uint16_t* Kc;
    const uint16_t* Vc;
    int page_size, num_pages, max_pages, Lmax;
    int page_shift;  // log2(page_size) when it is a power of two
    const int* page_table;
    const int* ctx_len;
    const uint16_t* Kd;
    const uint16_t* Vd;
    int dsb, dss, dsh;
    void* O;
    int osb, oss, osh;
    int o_f32;
    float* LSE;
    float* part_o;
    float* part_lse;
    int* units_before;  // [0]: total weighted units W; [1 + b]: weighted units of the sequences before b
    int B, S, Hq, Hkv, G, n_rb, has_den, n_seg;
    int pe;  // extra units counted at the start of every pair (its piece-start cost)
    float c_log2;  // softmax_scale * log2(e)
    int* dbg;  // debug mode: TT_DEBUG_* bits of the out-of-range data read, or null
};

typedef __attribute__((address_space(4))) const int const_int;

// branch weights for the block-frequency estimates the register allocator
// uses: the rare paths (piece ends, ragged tails, batch refills) are cold
#define TT_LIKELY(x) __builtin_expect(!!(x), 1)
#define TT_UNLIKELY(x) __builtin_expect(!!(x), 0)

// ctx_len is read through the constant address space: scalar loads
__device__ __forceinline__ int seq_len(const Args& a, const int* __restrict__ ctx_len, int b) {
    return ctx_len ? clamp_len(((const_int*)ctx_len)[b], a.Lmax) : 0;
}
__device__ __forceinline__ int units_for(const Args& a, int L) { return (L + kTile - 1) / kTile + a.has_den; }

// x of another lane by a DPP pattern (0 where the pattern names none or the
// row is masked off): a register move, no LDS round trip
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int x) {
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (all active): prefix sums
// within each row of 16 lanes by shifts of 1, 2, 4 and 8, then the total of row
// 0 added to row 1 and of row 2 to row 3 (broadcast of lanes 15 and 47), then
// that of rows 0-1 to rows 2 and 3 (broadcast of lane 31)
__device__ __forceinline__ int wave_incl_scan(int x, int) {
    x += dpp_move<0x111, 0xF>(x);  // row_shr:1
    x += dpp_move<0x112, 0xF>(x);  // row_shr:2
    x += dpp_move<0x114, 0xF>(x);  // row_shr:4
    x += dpp_move<0x118, 0xF>(x);  // row_shr:8
    x += dpp_move<0x142, 0xA>(x);  // row_bcast:15, rows 1 and 3
    x += dpp_move<0x143, 0xC>(x);  // row_bcast:31, rows 2 and 3
    return x;
}

// Segments are cut by weighted units: every pair with tiles counts its tiles
// plus pe extra units before its first tile, the cost of starting a piece
// (query rows, the epilogue of the piece before), so that a segment holding
// piece starts gets fewer tiles. Tile t of a pair that starts at weighted unit
// V sits at V + pe + t.
//
// Per wave, with no LDS or barrier (every wave of the block gets the same
// result): the tiles of segment `seg`, n of them from tile t0 of pair pl0 of
// sequence b0; with `before` set, also the total weighted units and every
// sequence's first weighted unit there. ctx_len is read 64 sequences at a time.
__device__ void scan_segment(const Args& a, const int* __restrict__ ctx_len, int seg, int& n, int& b0, int& pl0,
                             int& t0, int* before) {
    const int lane = threadIdx.x & 63;
    const int mult = a.Hkv * a.n_rb;
    auto units_at = [&](int b) {  // tiles per pair of sequence b
        return b < a.B ? units_for(a, ctx_len ? clamp_len(ctx_len[b], a.Lmax) : 0) : 0;
    };
    auto weighted = [&](int u) { return u > 0 ? mult * (u + a.pe) : 0; };
    const int u_first = units_at(lane);
    int wv = 0;
    for (int base = 0; base < a.B; base += 64)
        wv += __builtin_amdgcn_readlane(wave_incl_scan(weighted(base == 0 ? u_first : units_at(base + lane)), lane), 63);
    const int len = (wv + a.n_seg - 1) / a.n_seg;
    const int x0 = seg * len, x1 = min(wv, x0 + len);
    // r0, r1: tiles before weighted units x0 and x1
    int r0 = -1, r1 = -1;
    b0 = pl0 = t0 = 0;
    int vcarry = 0, rcarry = 0;
    for (int base = 0; base < a.B; base += 64) {
        const int u = base == 0 ? u_first : units_at(base + lane);
        const int vu = weighted(u);
        const int vincl = vcarry + wave_incl_scan(vu, lane), vexcl = vincl - vu;
        const int rincl = rcarry + wave_incl_scan(mult * u, lane), rexcl = rincl - mult * u;
        if (before && base + lane < a.B) before[1 + base + lane] = vexcl;
        const unsigned long long h0 = __builtin_amdgcn_ballot_w64(vu > 0 && x0 >= vexcl && x0 < vincl);
        if (h0) {
            const int l = __builtin_ctzll(h0);
            const int ub = __builtin_amdgcn_readlane(u, l);
            const int off = x0 - __builtin_amdgcn_readlane(vexcl, l);
            b0 = base + l;
            pl0 = off / (ub + a.pe);
            t0 = max(off % (ub + a.pe) - a.pe, 0);
            r0 = __builtin_amdgcn_readlane(rexcl, l) + pl0 * ub + t0;
        }
        const unsigned long long h1 = __builtin_amdgcn_ballot_w64(vu > 0 && x1 >= vexcl && x1 < vincl);
        if (h1) {
            const int l = __builtin_ctzll(h1);
            const int ub = __builtin_amdgcn_readlane(u, l);
            const int off = x1 - __builtin_amdgcn_readlane(vexcl, l);
            r1 = __builtin_amdgcn_readlane(rexcl, l) + (off / (ub + a.pe)) * ub + max(off % (ub + a.pe) - a.pe, 0);
        }
        vcarry = __builtin_amdgcn_readlane(vincl, 63);
        rcarry = __builtin_amdgcn_readlane(rincl, 63);
        if (r1 >= 0 && !before) break;
    }
    if (r1 < 0) r1 = rcarry;  // x1 is the end of the stream
    n = r0 < 0 ? 0 : r1 - r0;
    if (before && lane == 0) before[0] = wv;
}

// Position in the tile stream. Pair pl of sequence b is (kv head g, row block
// pl - g*n_rb); its tiles are the prefix tiles t < units - has_den, then the
// block-key tile.
struct Cur {
    int b, pl, t;  // sequence, pair index within the sequence (g*n_rb + rb), tile within the pair
    int L, units;  // prefix length, tiles per pair of sequence b
    int g;         // kv head of pair pl
};

__device__ __forceinline__ bool is_prefix(const Cur& c, const Args& a) { return c.t < c.units - a.has_den; }

__device__ __forceinline__ void set_seq(Cur& c, const Args& a, const int* __restrict__ ctx_len, int b) {
    c.b = b;
    c.L = seq_len(a, ctx_len, b);
    c.units = (c.L + kTile - 1) / kTile + a.has_den;
}

__device__ __forceinline__ void set_pair(Cur& c, const Args& a, int pl) {
    c.pl = pl;
    c.g = pl / a.n_rb;
}

__device__ __forceinline__ void advance(Cur& c, const Args& a, const int* __restrict__ ctx_len) {
    if (TT_LIKELY(++c.t < c.units)) return;
    c.t = 0;
    if (c.pl + 1 < a.Hkv * a.n_rb) {
        set_pair(c, a, c.pl + 1);
        return;
    }
    set_pair(c, a, 0);
    for (;;) {
        if (c.b + 1 >= a.B) { c.units = 1; return; }
        set_seq(c, a, ctx_len, c.b + 1);
        if (c.units > 0) return;
    }
}

// j / page_size and j % page_size, by shifts when page_size is a power of two
template <bool P2>
__device__ __forceinline__ int page_of(const Args& a, int j) { return P2 ? (j >> a.page_shift) : j / a.page_size; }
template <bool P2>
__device__ __forceinline__ int slot_of(const Args& a, int j) {
    return P2 ? (j & (a.page_size - 1)) : j % a.page_size;
}

// Workgroup barrier ordering LDS accesses only: waits for this wave's own LDS
// reads and writes (lgkmcnt), not for the global loads in flight. The callers
// wait for the direct-to-LDS loads whose data other waves read next
// (vmcnt) just before it. The empty asm statements keep the compiler from
// moving memory accesses across, the scheduling barriers every other
// instruction.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 lds16(const uint8_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element i%4 of the 8-byte rows read by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ i16x4 lds_tr(const uint8_t* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// (x of this lane, x of lane l ^ 32), in some order: v_permlane32_swap
// exchanges the upper 32 lanes of its first operand with the lower 32 lanes of
// its second, so with x in both each lane ends up holding both values. Written
// in assembly because the compiler's model of the builtin's second result is
// wrong (it reads both results from one register). The s_nop pairs give the
// wait states a VALU write needs before a permlane reads it, and after.
__device__ __forceinline__ void with_partner(float x, float& p0, float& p1) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    p0 = __builtin_bit_cast(float, a);
    p1 = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float max_with_partner(float x) {
    float p0, p1;
    with_partner(x, p0, p1);
    return fmaxf(p0, p1);
}
__device__ __forceinline__ float sum_with_partner(float x) {
    float p0, p1;
    with_partner(x, p0, p1);
    return p0 + p1;
}

// This lane's index, computed where it is used: a value the compiler cannot
// hoist, so no per-lane address derived from it stays live across a loop
// (where it could be spilled, and the reload would wait for every load in
// flight).
__device__ __forceinline__ unsigned lane_here() {
    unsigned ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    return ln;
}

// The query fragments of a piece from their LDS copy (k-step ds of lane l at
// base + 16 l + 1024 ds). Read in assembly, with the wait for the reads
// inside: the copy was written by direct-to-LDS loads whose completion the
// caller has already waited for, and the compiler, which cannot see that,
// would wait for every load in flight before the reads.
template <int DS>
__device__ __forceinline__ void read_q_lds(bf16x8 (&qf)[DS], unsigned base) {
    const unsigned addr = base + 16 * lane_here();
    u32x4 r[DS];
    if constexpr (DS == 8) {
        asm volatile(
            "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:1024\n\tds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\tds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
            "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
            : "v"(addr)
            : "memory");
    } else {
        static_assert(DS == 4, "");
        asm volatile(
            "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\tds_read_b128 %2, %4 offset:2048\n\t"
            "ds_read_b128 %3, %4 offset:3072\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
            : "v"(addr)
            : "memory");
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[ds] = __builtin_bit_cast(bf16x8, r[ds]);
}

// Sixteen bytes per lane from each of four LDS addresses, and an 8-byte LDS
// write: in assembly for the same reason (the buffer they use also receives
// direct-to-LDS loads, none of them in flight when these run). The reads wait
// for themselves and for every LDS access before them.
__device__ __forceinline__ void lds_read_x4(u32x4 (&r)[4], const unsigned (&ad)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
}
__device__ __forceinline__ void lds_write_b64(unsigned addr, unsigned lo, unsigned hi) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = {lo, hi};
    asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// ---- tile staging: global -> LDS ------------------------------------------
// Wave wq (0..3 within its group) moves keys 16 wq .. 16 wq + 15 of its
// group's half tile with LPG direct-to-LDS buffer loads of 1 KB: load k
// writes tile rows 16 wq + RPI k + lane / CPR, the lane's 16 bytes at slot
// lane % CPR of the row, which holds global chunk (lane % CPR) ^ swizzle.
// Sixteen 16-aligned keys lie in one page, so one page id serves the wave for
// the whole tile, and a full block reads 16 contiguous rows of that page.
// goff[k] is the lane's byte offset for load k of a full block; load k writes
// LDS from lbuf + (16 wq + RPI k) * ROWB = lbuf + 16 wq * ROWB + 1024 k.
template <int D>
__device__ __forceinline__ unsigned stage_chunk(bool v_half, int r, int p) {
    return v_half ? (unsigned)(p ^ (vswz<D>(r) << 2)) : (unsigned)(p ^ kswz<D>(r));
}

// Issue this wave's loads of tile c into LDS buffer `lbuf`. The prefix block is
// read through a buffer resource covering its 16 rows only. A block that
// reaches past the prefix end reads its last key again in the rows beyond it
// (finite data, weight exactly 0); a block wholly past the end reads the block
// holding the last key. A page id outside [0, num_pages) is clamped, so a
// corrupt table reads wrong data but never faults.
template <int D, bool P2>
__device__ __forceinline__ void dma_tile(uint8_t* lbuf, const Cur& c, int page, const uint16_t* src_c,
                                         const uint16_t* src_d, const Args& a, bool v_half, int wq,
                                         const unsigned (&goff)[Cfg<D>::LPG]) {
    using C = Cfg<D>;
    __amdgpu_buffer_rsrc_t rs;
    unsigned off[C::LPG];
    if (TT_LIKELY(is_prefix(c, a))) {
        int j0 = c.t * kTile + 16 * wq;
        if (TT_UNLIKELY(j0 >= c.L)) j0 = (c.L - 1) & ~15;
        const int last = c.L - 1 - j0;  // rows 0..last of the block are keys
        page = min(max(page, 0), a.num_pages - 1);
        const uint16_t* base = src_c + (((long long)page * a.Hkv + c.g) * a.page_size + slot_of<P2>(a, j0)) * D;
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 16 * C::ROWB, 0x00020000);
        if (TT_LIKELY(last >= 15)) {
#pragma unroll
            for (int k = 0; k < C::LPG; ++k) off[k] = goff[k];
        } else {
            const unsigned ln = lane_here();
#pragma unroll
            for (int k = 0; k < C::LPG; ++k) {
                const int rr = C::RPI * k + (int)(ln / C::CPR);
                off[k] = (unsigned)(min(rr, last) * C::ROWB) + 16u * stage_chunk<D>(v_half, rr, (int)(ln % C::CPR));
            }
        }
    } else {
        const uint16_t* base = src_d + (long long)c.b * a.dsb + (long long)c.g * a.dsh;
        rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
        const unsigned ln = lane_here();
#pragma unroll
        for (int k = 0; k < C::LPG; ++k) {
            const int rr = C::RPI * k + (int)(ln / C::CPR);
            off[k] = (unsigned)(min(16 * wq + rr, a.S - 1) * a.dss * 2) +
                     16u * stage_chunk<D>(v_half, rr, (int)(ln % C::CPR));
        }
    }
    uint8_t* const dst = lbuf + 16 * wq * C::ROWB;
    // With one row block per (sequence, kv head) every K/V byte is read once: the loads
    // are non-temporal (nt), so the stream does not displace cached data. With more
    // row blocks the other blocks read the same tiles, and the caches may still hold them.
    if (a.n_rb == 1) {
#pragma unroll
        for (int k = 0; k < C::LPG; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 1024 * k),
                                                     16, off[k], 0, 0, 2);
    } else {
#pragma unroll
        for (int k = 0; k < C::LPG; ++k)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 1024 * k),
                                                     16, off[k], 0, 0, 0);
    }
}

template <int D, bool P2>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(Args a, const int* __restrict__ page_table,
                                                                const int* __restrict__ ctx_len) {
    using C = Cfg<D>;
    // K and V tiles, two buffers each (tile j in buffer j % 2). Separate
    // arrays, so that the compiler tells the buffers apart when it places the
    // waits for the direct-to-LDS loads before its own LDS reads.
    __shared__ __attribute__((aligned(1024))) uint8_t kb0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t kb1[C::TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t vb0[C::TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t vb1[C::TILEB];
    __shared__ int pgs[kWaves][2][64];  // page-id batches of each wave
    // Query rows of the next piece, fetched ahead: wave w's 32 rows, lane l's
    // 16 bytes of k-step ds at [w][1024 ds + 16 l]. Between pieces the same
    // bytes stage a finished piece's bf16 rows (32 rows of pitch ROWB + 16).
    __shared__ __attribute__((aligned(16))) uint8_t qlds[kWaves][C::DS * 1024 + 512];
    uint8_t* const KR[2] = {kb0, kb1};
    uint8_t* const VR[2] = {vb0, vb1};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = wave & 3;
    const bool vh = wave >= 4;  // this wave loads the V half of every tile
    const int l32 = lane & 31, hl = lane >> 5;

    // logical segment of this workgroup: consecutive segments share an XCD
    const int per_xcd = a.n_seg / 8;
    const int seg = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;

    if (TT_UNLIKELY(a.dbg != nullptr) && ctx_len && blockIdx.x == 0 && wave == 0) {
        bool bad = false;
        for (int b = lane; b < a.B; b += 64) bad |= ctx_len[b] < 0 || ctx_len[b] > a.Lmax;
        if (bad) atomicOr(a.dbg, TT_DEBUG_CTX_LEN);
    }
    int n, b0, pl0, t0;  // tiles of this segment, from tile t0 of pair pl0 of sequence b0
    scan_segment(a, ctx_len, seg, n, b0, pl0, t0, seg == 0 && wave == 0 ? a.units_before : nullptr);
    n = __builtin_amdgcn_readfirstlane(n);
    if (n <= 0) return;
    b0 = __builtin_amdgcn_readfirstlane(b0);
    pl0 = __builtin_amdgcn_readfirstlane(pl0);
    t0 = __builtin_amdgcn_readfirstlane(t0);
    if (TT_UNLIKELY(a.dbg != nullptr)) {
        // Debug mode: every LDS byte starts as all ones (a NaN in bf16, page id -1), so a
        // read of LDS that no load or store of this call filled reaches the outputs or the
        // flags. The barrier orders the fill before any wave's first load into LDS.
        auto poison = [&](void* p, int bytes) __attribute__((always_inline)) {
            for (int o = tid * 16; o < bytes; o += kThreads * 16)
                *reinterpret_cast<u32x4*>(static_cast<uint8_t*>(p) + o) = u32x4{~0u, ~0u, ~0u, ~0u};
        };
        poison(kb0, C::TILEB);
        poison(kb1, C::TILEB);
        poison(vb0, C::TILEB);
        poison(vb1, C::TILEB);
        poison(pgs, (int)sizeof(pgs));
        poison(qlds, (int)sizeof(qlds));
        lds_barrier();
    }

    Cur cc;  // tile being computed
    set_seq(cc, a, ctx_len, b0);
    set_pair(cc, a, pl0);
    cc.t = t0;
    const int mult = a.Hkv * a.n_rb;

    // ---- this wave's half of every tile ----
    const uint16_t* src_c = vh ? a.Vc : a.Kc;
    const uint16_t* src_d = vh ? a.Vd : a.Kd;
    // this lane's byte offsets for the loads of a full 16-key block
    unsigned goff[C::LPG];
#pragma unroll
    for (int k = 0; k < C::LPG; ++k)
        goff[k] = (unsigned)((C::RPI * k + lane / C::CPR) * C::ROWB) +
                  16u * stage_chunk<D>(vh, C::RPI * k + lane / C::CPR, lane % C::CPR);
    // page ids through a bounds-checked buffer resource (an empty table reads 0)
    const __amdgpu_buffer_rsrc_t ptab = __builtin_amdgcn_make_buffer_rsrc(
        (void*)page_table, (short)0, page_table ? a.B * a.max_pages * 4 : 0, 0x00020000);

    // Page ids come in batches of 64 tiles, double-buffered in LDS: lane l
    // walks the tile stream from cursor c (tile `first` of the segment) by
    // ahead + l tiles (across pair and sequence boundaries) and fetches the
    // page of its 16 keys with one direct-to-LDS buffer load for the batch. A
    // batch is fetched when the one before it comes into use, 64 tiles ahead
    // of its own first use.
    auto page_batch = [&](const Cur& c, int first, int ahead, int buf) __attribute__((always_inline)) {
        int idx = 0;
        if (lane + ahead < n - first) {  // tiles past the segment stay at index 0
            int b = c.b, pl = c.pl, t = c.t + ahead + lane, L = c.L, units = c.units;
            while (t >= units) {
                t -= units;
                if (++pl == mult) {
                    pl = 0;
                    do {
                        ++b;
                        L = seq_len(a, ctx_len, b);
                        units = (L + kTile - 1) / kTile + a.has_den;
                    } while (units == 0);
                }
            }
            if (t < units - a.has_den) idx = b * a.max_pages + page_of<P2>(a, min(t * kTile + 16 * wq, L - 1));
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ptab, (__attribute__((address_space(3))) void*)&pgs[wave][buf][0], 4,
                                                 idx * 4, 0, 0, 0);
    };

    // Direct-to-LDS copy of the query rows of the piece at c (the fragments
    // load_q would read, each lane's 16 bytes of step ds at qlds[wave][1024 ds +
    // 16 lane]). It is issued when the load cursor enters the piece, if the
    // buffer is free.
    auto q_dma = [&](const Cur& c) __attribute__((always_inline)) {
        const unsigned ln = lane_here();
        const int rb = c.pl - c.g * a.n_rb;
        const int rr = min(rb * kRows + wave * 32 + (int)(ln & 31), a.S * a.G - 1);
        const int s = rr / a.G, h = c.g * a.G + rr % a.G;
        const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(a.Q + (long long)c.b * a.qsb), (short)0, 0x7FFFFFFF, 0x00020000);
        const int off = (s * a.qss + h * a.qsh + (int)(ln >> 5) * 8) * 2;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (__attribute__((address_space(3))) void*)&qlds[wave][ds * 1024], 16,
                                                     off + ds * 32, 0, 0, 0);
    };
    int q_tag = -1;  // segment index of the piece start whose rows are in qlds (-1: none)

    // Load pipeline: the K waves request tile i+1 and the V waves tile i at
    // the start of tile i's phase (V is used one tile later than K), and every
    // wave waits for its own loads before the barrier that ends the phase.
    // Every issue loads a whole tile; once the segment's last tile is loaded
    // (the K waves get there a phase before the V waves) an issue loads
    // nothing, and the waits on vmcnt(0) need no count.
    Cur cl = cc;  // next tile to load
    int ul = 0;   // its index in the segment
    bool all_loaded = false;
    int pg_base = 0;
    // The batch in use is also kept in a register (lane l: tile pg_base + l),
    // so a tile's id is a readlane and its LDS copy is read once per batch.
    int pbuf = 0;  // batch in use
    page_batch(cl, 0, 0, 0);
    page_batch(cl, 0, 64, 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): both batches have landed
    int pgl = pgs[wave][0][lane];
    auto issue = [&](uint8_t* lbuf) __attribute__((always_inline)) {
        if (TT_UNLIKELY(ul - pg_base == 64)) {
            pg_base = ul;
            pbuf ^= 1;
            pgl = pgs[wave][pbuf][lane];
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): here, not before every tile's readlane
            page_batch(cl, ul, 64, pbuf ^ 1);    // the batch after next, into the one used up
        }
        if (TT_UNLIKELY(all_loaded)) return;
        const int page = __builtin_amdgcn_readlane(pgl, ul - pg_base);
        if (TT_UNLIKELY(a.dbg != nullptr) && is_prefix(cl, a) && (page < 0 || page >= a.num_pages) && lane == 0)
            atomicOr(a.dbg, TT_DEBUG_PAGE_ID);
        dma_tile<D, P2>(lbuf, cl, page, src_c, src_d, a, vh, wq, goff);
        if (ul + 1 < n) {
            advance(cl, a, ctx_len);
            ++ul;
            if (TT_UNLIKELY(cl.t == 0 && q_tag < 0)) {
                q_dma(cl);
                q_tag = ul;
            }
        } else {
            all_loaded = true;
        }
    };

    // ---- per-wave state ----
    bf16x8 qf[C::DS];
    f32x16 oacc[C::DT];
    f32x16 sacc[2][2];  // scores of tile j in sacc[j % 2]
    bf16x8 pf[4];
    float m2 = -INFINITY, lsum = 0.f;
    int piece_t0 = 0;
    // lane parts of the LDS operand addresses. Score reads take chunk 2 cc + hl
    // of row l32 (+32 mt): kad[cc]. V reads take bytes 64 dt + vin of row vr
    // (+16 ks, +8 for the second half): vad[dt]. The swizzles of rows l32 + 32 mt
    // and vr + 16 ks + 8 are those of l32 and vr.
    unsigned kad[C::DS], vad[C::DT];
#pragma unroll
    for (int c2 = 0; c2 < C::DS; ++c2) kad[c2] = l32 * C::ROWB + 16 * ((2 * c2 + hl) ^ kswz<D>(l32));
    {
        const int vr = 4 * hl + ((lane & 15) >> 2);
        const int vin = 16 * (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) + 8 * (lane & 1);
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) vad[dt] = vr * C::ROWB + 64 * (dt ^ vswz<D>(vr)) + vin;
    }

    // query rows of the pair at c (a row past S*G reads the last row; it is never written)
    auto load_q = [&](const Cur& c) __attribute__((always_inline)) {
        const unsigned ln = lane_here();
        const int rb = c.pl - c.g * a.n_rb;
        const int rr = min(rb * kRows + wave * 32 + (int)(ln & 31), a.S * a.G - 1);
        const int s = rr / a.G, h = c.g * a.G + rr % a.G;
        const uint16_t* q =
            a.Q + (long long)c.b * a.qsb + (long long)s * a.qss + (long long)h * a.qsh + (int)(ln >> 5) * 8;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) qf[ds] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + ds * 16));
    };

    // matrix part of tile j: S^T of tile j from K buffer KB = j % 2 into
    // sacc[KB] (if QK); the softmax of tile j-1 (scores sacc[VB], running max
    // from the tile before) and O^T += V^T P^T for it from V buffer VB =
    // (j-1) % 2 (if PV). Per 16-key step ks: the operands of step ks+1 are
    // read from LDS while the step's MFMAs run, and the softmax of keys
    // 16ks .. 16ks+15 (P^T fragment pf[ks]) fills the vector ALU meanwhile.
    // The score product runs K-row half outer (steps 0-1 rows 0-31, steps 2-3
    // rows 32-63), so the new tile's second half comes alive as the old
    // tile's first half is used up.
    constexpr int DPS = C::DS / 2;  // d steps of the score product per step
    struct Frag {
        bf16x8 k[DPS];
        bf16x8 v[C::DT];
    };
    auto matrix = [&](auto QK_, auto PV_, auto KB_, auto VB_) __attribute__((always_inline)) {
        constexpr bool QK = decltype(QK_)::value;
        constexpr bool PV = decltype(PV_)::value;
        constexpr int KB = decltype(KB_)::value, VB = decltype(VB_)::value;
        const uint8_t* Kst = KR[KB];
        const uint8_t* Vst = VR[VB];
        auto read = [&](Frag& f, auto KS_) __attribute__((always_inline)) {
            constexpr int ks = decltype(KS_)::value;
            if constexpr (QK) {
#pragma unroll
                for (int dd = 0; dd < DPS; ++dd)
                    f.k[dd] = lds16(Kst + kad[(ks % 2) * DPS + dd] + (ks / 2) * 32 * C::ROWB);
            }
            if constexpr (PV) {
                // V sits in LDS as [key][d]; the transposing read hands lane l the four keys
                // kb..kb+3 of column d = 32*dt + l%32, with kb = 16*ks + 8*half + 4*(l/32):
                // exactly the keys its P^T slots hold.
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const uint8_t* p0 = Vst + vad[dt] + ks * 16 * C::ROWB;
                    const i16x4 pair[2] = {lds_tr(p0), lds_tr(p0 + 8 * C::ROWB)};
                    f.v[dt] = __builtin_bit_cast(bf16x8, pair);
                }
            }
        };
        const float neg = -m2;
        float ls = 0.f;
        auto step = [&](const Frag& f, auto KS_) __attribute__((always_inline)) {
            constexpr int ks = decltype(KS_)::value;
            if constexpr (PV) {
                f32x8 pv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[VB][ks >> 1][(ks & 1) * 8 + e], a.c_log2, neg));
                    ls += pv[e];
                }
                pf[ks] = __builtin_convertvector(pv, bf16x8);
            }
            if constexpr (QK) {
                constexpr int mt = ks / 2;
#pragma unroll
                for (int dd = 0; dd < DPS; ++dd)
                    sacc[KB][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        f.k[dd], qf[(ks % 2) * DPS + dd], (ks % 2 == 0 && dd == 0) ? f32x16{} : sacc[KB][mt], 0, 0,
                        0);
            }
            if constexpr (PV) {
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.v[dt], pf[ks], oacc[dt], 0, 0, 0);
            }
        };
        auto interleave = []() __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // LDS read
            }
        };
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        Frag f0, f1;
        read(f0, I0{});
        read(f1, I1{});
        step(f0, I0{});
        __builtin_amdgcn_sched_barrier(0);
        // in the two middle regions, pairs of MFMAs alternate with groups of three
        // LDS reads
        read(f0, I2{});
        step(f1, I1{});
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        read(f1, I3{});
        step(f0, I2{});
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        step(f1, I3{});
        if constexpr (PV) lsum += ls;
    };

    // A finished piece of pair pl of sequence b: the normalised output if the
    // piece is the whole pair, else a partial for the merge kernel. oacc is
    // scaled in place (the caller resets it next).
    auto epilogue = [&](int b, int pl, int g, bool full) __attribute__((always_inline)) {
        const float lt = sum_with_partner(lsum);
        const float inv = 1.f / lt;
        const float lse = (m2 + __log2f(lt)) * kLn2;
        const int rl = wave * 32 + l32;  // row within the block
        const int rb = pl - g * a.n_rb;
        const int rr = rb * kRows + rl;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[dt][e] *= inv;
        if (!full && !a.o_f32 && q_tag < 0) {
            // A partial in bf16: the rows go through this wave's query buffer (its
            // rows have been read and no copy is in flight), so that every store
            // writes whole rows (a lane holds 8-byte pieces of one row). The
            // padded pitch spreads the writes over the banks.
            const unsigned ln = lane_here();
            constexpr int SP = C::ROWB + 16;
            const unsigned qb = (unsigned)(uintptr_t)&qlds[wave][0];
            const unsigned wa = qb + (ln & 31) * SP + ((ln >> 5) << 3);
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 v = __builtin_bit_cast(
                        u32x2, __builtin_convertvector((f32x4{oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2],
                                                              oacc[dt][4 * j + 3]}),
                                                       bf16x4));
                    lds_write_b64(wa + ((4 * dt + j) << 4), v[0], v[1]);
                }
            // lane l now takes chunk l % CPR of rows RPI*k + l / CPR; a wave's 32
            // rows of the slot are 32*D contiguous elements
            constexpr int NK = 32 / C::RPI;
            const unsigned ra0 = qb + (ln / C::CPR) * SP + ((ln % C::CPR) << 4);
            const long long slot = seg + b * mult + pl;
            char* const po = reinterpret_cast<char*>(a.part_o) + (slot * kRows + wave * 32) * (D * 2);
#pragma unroll
            for (int k0 = 0; k0 < NK; k0 += 4) {
                unsigned ra[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) ra[k] = ra0 + C::RPI * (k0 + k) * SP;
                u32x4 v[4];
                lds_read_x4(v, ra);
#pragma unroll
                for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(po + (ln * 16 + (k0 + k) * 1024)) = v[k];
            }
            if ((ln >> 5) == 0 && (rb * kRows + wave * 32 + (int)(ln & 31)) < a.S * a.G)
                *reinterpret_cast<float*>(reinterpret_cast<char*>(a.part_lse) + (slot * kRows + wave * 32) * 4 +
                                          (ln & 31) * 4) = lse;
            return;
        }
        if (rr >= a.S * a.G) return;
        // lane holds d = 32*dt + 8*j + 4*hl + (0..3) in oacc[dt][4j .. 4j+3]
        if (full) {
            const int s = rr / a.G, h = g * a.G + rr % a.G;
            const long long ob = (long long)b * a.osb + (long long)s * a.oss + (long long)h * a.osh + hl * 4;
            if (a.o_f32) {
                float* o = reinterpret_cast<float*>(a.O) + ob;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<f32x4*>(o + dt * 32 + j * 8) =
                            f32x4{oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]};
            } else {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                __bf16* o = reinterpret_cast<__bf16*>(a.O) + ob;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<bf16x4*>(o + dt * 32 + j * 8) = __builtin_convertvector(
                            (f32x4{oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]}),
                            bf16x4);
            }
            if (a.LSE && hl == 0) a.LSE[((long long)b * a.Hq + h) * a.S + s] = lse;
        } else {
            // partial O in the output's precision: fp32 for an fp32 output, else bf16
            const long long slot = seg + b * mult + pl;
            const long long pe = (slot * kRows + rl) * D + hl * 4;
            if (a.o_f32) {
                float* po = a.part_o + pe;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<f32x4*>(po + dt * 32 + j * 8) =
                            f32x4{oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]};
            } else {
                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                __bf16* po = reinterpret_cast<__bf16*>(a.part_o) + pe;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<bf16x4*>(po + dt * 32 + j * 8) = __builtin_convertvector(
                            (f32x4{oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]}),
                            bf16x4);
            }
            if (hl == 0) a.part_lse[slot * kRows + rl] = lse;
        }
    };

    // the piece of tile i - 1, if that tile ended its pair
    bool prev_ends = false;
    int prev_b = 0, prev_pl = 0, prev_g = 0;
    // vector part of tile i: close the piece that ended with tile i-1 (its last
    // softmax and PV product ran in this tile's matrix part), mask and row max
    // of tile i (the rescale it may call for applies before tile i's weights
    // are added, in the next matrix part), move to tile i+1
    auto vector = [&](auto P_, int i) __attribute__((always_inline)) {
        constexpr int P = decltype(P_)::value;  // i % 2
        const bool close_prev = i > 0 && prev_ends;
        if (TT_UNLIKELY(close_prev)) epilogue(prev_b, prev_pl, prev_g, piece_t0 == 0);
        if (TT_UNLIKELY(i == 0 || close_prev)) {
            piece_t0 = cc.t;
            m2 = -INFINITY;
            lsum = 0.f;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][e] = 0.f;
        }
        const int nvalid = is_prefix(cc, a) ? min(kTile, cc.L - cc.t * kTile) : a.S;
        if (TT_UNLIKELY(nvalid < kTile)) {
            // key of element e of sacc[mt] is mt*32 + 8*(e/4) + e%4 + 4*hl
            const int lim = nvalid - 4 * hl;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (mt * 32 + (e >> 2) * 8 + (e & 3) >= lim) sacc[P][mt][e] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[P][mt][e]);
        const float mnew = max_with_partner(mx) * a.c_log2;
        const bool need = mnew > m2 + kTau;
        if (TT_UNLIKELY(__builtin_amdgcn_ballot_w64(need))) {
            const float alpha = need ? __builtin_amdgcn_exp2f(m2 - mnew) : 1.f;
            if (need) m2 = mnew;
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[dt][e] *= alpha;
        }
        // next tile: its query rows if it starts a new piece
        prev_ends = cc.t == cc.units - 1;
        prev_b = cc.b;
        prev_pl = cc.pl;
        prev_g = cc.g;
        if (i + 1 < n) {
            advance(cc, a, ctx_len);
            if (TT_UNLIKELY(cc.t == 0)) {
                if (q_tag == i + 1) {
                    // the copy may still be in flight (a V wave issues it in this tile)
                    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                    read_q_lds(qf, (unsigned)(uintptr_t)&qlds[wave][0]);
                    q_tag = -1;
                } else {
                    load_q(cc);
                    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
                }
            }
        }
    };

    // One phase per tile i: the loads (K of tile i+1, V of tile i), the matrix
    // part (scores of i, softmax and PV of i-1), the vector part, then this
    // wave's loads are waited for and the barrier hands the buffers over.
    using F = std::false_type;
    using T = std::true_type;
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    auto tile = [&](auto J_, int i) __attribute__((always_inline)) {
        constexpr int J = decltype(J_)::value;  // i % 2
        using JC = std::integral_constant<int, J>;
        using JP = std::integral_constant<int, 1 - J>;
        issue(vh ? VR[J] : KR[1 - J]);
        matrix(T{}, T{}, JC{}, JP{});
        vector(JC{}, i);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's part of tile i+1 (K) / i (V)
        lds_barrier();
    };

    // ---- prologue: K of tile 0 and the query rows of the first piece ----
    if (!vh) issue(KR[0]);
    load_q(cc);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    lds_barrier();
    // tile 0: no PV product yet
    issue(vh ? VR[0] : KR[1]);
    matrix(T{}, F{}, Z{}, O{});
    vector(Z{}, 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();
    int i = 1;
    for (; i + 1 < n; i += 2) {
        tile(O{}, i);
        tile(Z{}, i + 1);
    }
    if (i < n) {
        tile(O{}, i);
        ++i;
    }
    // PV of the last tile, n - 1
    if ((n - 1) % 2 == 0)
        matrix(F{}, T{}, Z{}, Z{});
    else
        matrix(F{}, T{}, Z{}, O{});
    epilogue(cc.b, cc.pl, cc.g, piece_t0 == 0 && cc.t == cc.units - 1);
}

// Merge the per-segment partials of every pair that segment boundaries cut,
// and write O = 0, LSE = -inf for pairs with no keys at all. The pair's
// segments follow from the unit counts the main kernel left in the workspace.
// Grid: n_pairs * (kRows / RPW) workgroups of PS thread groups of 16 RPW
// threads, RPW rows each; a row's 16 threads take D/16 consecutive elements
// each. Partials are read eight at a time, every load of a group issued before
// any is used, and the next group is in flight while one is merged. With PS > 1
// (pairs cut into many pieces) thread group q of the workgroup takes every
// PS-th partial from the q-th, and group 0 merges the groups' results from LDS
// in group order; so a pair cut into many segments costs few memory round
// trips (with eight groups, up to 64 partials in one).
template <int D, bool F32, int PS, int RPW>
__global__ __launch_bounds__(16 * RPW * PS) void attn_bf16_finalize(Args a, const int* __restrict__ ctx_len) {
    constexpr int GT = 16 * RPW;            // threads per group
    constexpr int CH = kRows / RPW;         // workgroups per pair
    constexpr int EPT = D / 16;             // elements per thread
    constexpr int NG = F32 && PS > 1 ? 4 : 8;  // partials per group (fp32 ones in four at most 128 registers)
    const int mult = a.Hkv * a.n_rb;
    const int p = blockIdx.x / CH, chunk = blockIdx.x % CH;
    const int b = p / mult, pl = p % mult;
    const int g = pl / a.n_rb, rb = pl % a.n_rb;
    const int W = a.units_before[0];
    const int units = units_for(a, ctx_len ? clamp_len(ctx_len[b], a.Lmax) : 0);  // tiles per pair
    const int seg_len = (W + a.n_seg - 1) / a.n_seg;
    int s0 = 0, s1 = -1;
    if (units > 0) {
        // weighted unit of the pair's first tile
        const int U = a.units_before[1 + b] + pl * (units + a.pe) + a.pe;
        s0 = U / seg_len;
        s1 = (U + units - 1) / seg_len;
        if (s0 == s1) return;  // written by the main kernel
    }
    const int grp = threadIdx.x / GT;  // partial group (PS > 1)
    const int tid = threadIdx.x % GT;
    const int rl = chunk * RPW + tid / 16;  // row within the block
    const int rr = rb * kRows + rl;
    const bool live = rr < a.S * a.G;
    if (PS == 1 && !live) return;
    const int s = rr / a.G, h = g * a.G + rr % a.G;
    const long long ob = (long long)b * a.osb + (long long)s * a.oss + (long long)h * a.osh;
    const int d0 = (tid % 16) * EPT;
    typedef float f32xE __attribute__((ext_vector_type(EPT)));
    typedef __bf16 bf16xE __attribute__((ext_vector_type(EPT)));
    typedef typename std::conditional<F32, f32xE, bf16xE>::type raw_t;
    struct Group {
        float l[NG];
        raw_t v[NG];
    };
    // partials past s1 are not read (the bound is uniform over the thread group)
    auto load = [&](int sg0, Group& gr) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (sg0 + PS * j > s1) break;
            const long long slot = sg0 + PS * j + p;
            gr.l[j] = a.part_lse[slot * kRows + rl];
            const long long pe = (slot * kRows + rl) * D + d0;
            if constexpr (F32)
                gr.v[j] = *reinterpret_cast<const f32xE*>(a.part_o + pe);
            else
                gr.v[j] = *reinterpret_cast<const bf16xE*>(reinterpret_cast<const __bf16*>(a.part_o) + pe);
        }
    };
    float M = -INFINITY, Wsum = 0.f;
    f32xE acc = {};
    auto merge = [&](int sg0, const Group& gr) __attribute__((always_inline)) {
        float mg = M;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (sg0 + PS * j > s1) break;
            mg = fmaxf(mg, gr.l[j]);
        }
        if (mg == -INFINITY) return;
        const float sc = __expf(M - mg);  // 0 while M is -inf
        Wsum *= sc;
        acc *= sc;
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            if (sg0 + PS * j > s1) break;
            const float w = gr.l[j] != -INFINITY ? __expf(gr.l[j] - mg) : 0.f;
            Wsum += w;
            if constexpr (F32)
                acc += w * gr.v[j];
            else
                acc += w * __builtin_convertvector(gr.v[j], f32xE);
        }
        M = mg;
    };
    Group ga, gb;
    const int q0 = s0 + grp;  // this group's first partial
    constexpr int STEP = PS * NG;
    if (live && q0 <= s1) {
        load(q0, ga);
        for (int sg0 = q0; sg0 <= s1; sg0 += 2 * STEP) {
            if (sg0 + STEP <= s1) load(sg0 + STEP, gb);
            merge(sg0, ga);
            if (sg0 + STEP > s1) break;
            if (sg0 + 2 * STEP <= s1) load(sg0 + 2 * STEP, ga);
            merge(sg0 + STEP, gb);
        }
    }
    if constexpr (PS > 1) {
        // groups 1..PS-1 hand (M, Wsum, acc) to group 0, which merges them in group order
        __shared__ float xm[PS - 1][GT], xw[PS - 1][GT];
        __shared__ f32xE xa[PS - 1][GT];
        if (grp > 0) {
            xm[grp - 1][tid] = M;
            xw[grp - 1][tid] = Wsum;
            xa[grp - 1][tid] = acc;
        }
        __syncthreads();
        if (grp > 0 || !live) return;
#pragma unroll
        for (int q = 0; q < PS - 1; ++q) {
            const float mq = xm[q][tid];
            const float mg = fmaxf(M, mq);
            if (mg == -INFINITY) continue;
            const float sa = __expf(M - mg), sb = __expf(mq - mg);  // 0 for a side still at -inf
            Wsum = Wsum * sa + xw[q][tid] * sb;
            acc = acc * sa + xa[q][tid] * sb;
            M = mg;
        }
    }
    const float inv = Wsum > 0.f ? 1.f / Wsum : 0.f;
    const f32xE o = acc * inv;
    if (a.o_f32)
        *reinterpret_cast<f32xE*>(reinterpret_cast<float*>(a.O) + ob + d0) = o;
    else
        *reinterpret_cast<bf16xE*>(reinterpret_cast<__bf16*>(a.O) + ob + d0) = __builtin_convertvector(o, bf16xE);
    if (a.LSE && tid % 16 == 0)
        a.LSE[((long long)b * a.Hq + h) * a.S + s] = Wsum > 0.f ? M + __logf(Wsum) : -INFINITY;
}

// Scratch of the allocation-free entry point: the workspace of tt_block_attn,
// held by the library. Host code never passes this name to a kernel (on the
// host it is only a stand-in for the symbol); it uses the device address that
// noalloc_scratch() looks up once per device.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

}  // namespace

void* noalloc_scratch(tt_status* st) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
        *st = TT_ERR_HIP;
        return nullptr;
    }
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    // this device's copy of the array, looked up with the device current
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        *st = TT_ERR_HIP;
        return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

AttnPlan plan_attn_bf16(const tt_block_attn_params& p, int n_cu) {
    AttnPlan pl{};
    const int G = p.Hq / p.Hkv;
    pl.n_rb = (p.S * G + kRows - 1) / kRows;
    pl.n_pairs = p.B * p.Hkv * pl.n_rb;
    const long long tiles_max = (long long)(p.max_ctx_len + kTile - 1) / kTile + (p.Kden ? 1 : 0);
    const long long w_max = (long long)pl.n_pairs * tiles_max;
    const int cu8 = ((n_cu > 0 ? n_cu : 256) + 7) / 8 * 8;
    long long nseg = (w_max + 1) / 2;  // at least two tiles per segment
    nseg = (nseg + 7) / 8 * 8;
    if (nseg > cu8) nseg = cu8;
    if (nseg < 8) nseg = 8;
    pl.n_seg = (int)nseg;
    pl.n_slots = pl.n_seg + pl.n_pairs;
    // partial O is kept in the output's precision
    pl.ws_part_o = (size_t)pl.n_slots * kRows * p.head_dim * (p.o_dtype == TT_F32 ? 4 : 2);
    pl.ws_part_lse = (size_t)pl.n_slots * kRows * sizeof(float);
    pl.ws_units = ((size_t)(p.B + 1) * sizeof(int) + 255) / 256 * 256;
    pl.ws_total = pl.ws_part_o + pl.ws_part_lse + pl.ws_units + 256;
    // pairs cut into many pieces on average: the merge splits each pair's
    // partials over four thread groups (16 or more pieces), or eight of four rows
    // each (32 or more)
    pl.fin_split = (long long)pl.n_seg >= 32LL * pl.n_pairs ? 8 : ((long long)pl.n_seg >= 16LL * pl.n_pairs ? 4 : 1);
    return pl;
}

tt_status launch_attn_bf16(const tt_block_attn_params& p, const AttnPlan& pl, void* ws, hipStream_t s) {
    Args a{};
    a.Q = static_cast<const uint16_t*>(p.Q);
    a.qsb = (int)p.q_stride_b; a.qss = (int)p.q_stride_s; a.qsh = (int)p.q_stride_h;
    a.Kc = static_cast<const uint16_t*>(p.Kctx);
    a.Vc = static_cast<const uint16_t*>(p.Vctx);
    a.page_size = p.page_size; a.num_pages = p.num_pages; a.max_pages = p.max_pages;
    const long long cap = (long long)p.max_pages * p.page_size;
    a.Lmax = (int)(p.max_ctx_len < cap ? p.max_ctx_len : cap);
    a.page_table = p.max_ctx_len > 0 ? p.page_table : nullptr;
    a.ctx_len = p.max_ctx_len > 0 ? p.ctx_len : nullptr;
    a.Kd = static_cast<const uint16_t*>(p.Kden);
    a.Vd = static_cast<const uint16_t*>(p.Vden);
    a.dsb = (int)p.den_stride_b; a.dss = (int)p.den_stride_s; a.dsh = (int)p.den_stride_h;
    a.O = p.O;
    a.osb = (int)p.o_stride_b; a.oss = (int)p.o_stride_s; a.osh = (int)p.o_stride_h;
    a.o_f32 = p.o_dtype == TT_F32;
    a.LSE = p.LSE;
    char* w = static_cast<char*>(ws);
    a.part_o = reinterpret_cast<float*>(w);
    a.part_lse = reinterpret_cast<float*>(w + pl.ws_part_o);
    a.units_before = reinterpret_cast<int*>(w + pl.ws_part_o + pl.ws_part_lse);
    a.B = p.B; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.Hq / p.Hkv;
    a.n_rb = pl.n_rb;
    a.has_den = p.Kden ? 1 : 0;
    a.n_seg = pl.n_seg;
    a.pe = kPieceCost;
    a.c_log2 = p.softmax_scale * 1.44269504088896340736f;
    a.dbg = p.debug_flags;
    a.page_shift = -1;
    if (p.page_size > 0 && (p.page_size & (p.page_size - 1)) == 0) {
        a.page_shift = 0;
        while ((1 << a.page_shift) < p.page_size) ++a.page_shift;
    }
    const bool p2 = a.page_shift >= 0;
    const dim3 grid(pl.n_seg), blk(kThreads);
    auto merge = [&](auto D_) {
        constexpr int D = decltype(D_)::value;
        const dim3 g16(pl.n_pairs * (kRows / kFinRows)), g4(pl.n_pairs * (kRows / 4));
        if (pl.fin_split == 8) {
            if (a.o_f32) hipLaunchKernelGGL((attn_bf16_finalize<D, true, 8, 4>), g4, dim3(8 * 64), 0, s, a, a.ctx_len);
            else hipLaunchKernelGGL((attn_bf16_finalize<D, false, 8, 4>), g4, dim3(8 * 64), 0, s, a, a.ctx_len);
        } else if (pl.fin_split == 4) {
            if (a.o_f32) hipLaunchKernelGGL((attn_bf16_finalize<D, true, 4, kFinRows>), g16, dim3(4 * 16 * kFinRows), 0, s, a, a.ctx_len);
            else hipLaunchKernelGGL((attn_bf16_finalize<D, false, 4, kFinRows>), g16, dim3(4 * 16 * kFinRows), 0, s, a, a.ctx_len);
        } else {
            if (a.o_f32) hipLaunchKernelGGL((attn_bf16_finalize<D, true, 1, kFinRows>), g16, dim3(16 * kFinRows), 0, s, a, a.ctx_len);
            else hipLaunchKernelGGL((attn_bf16_finalize<D, false, 1, kFinRows>), g16, dim3(16 * kFinRows), 0, s, a, a.ctx_len);
        }
    };
    if (p.head_dim == 128) {
        if (p2) hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        else hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        merge(std::integral_constant<int, 128>{});
    } else {
        if (p2) hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        else hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        merge(std::integral_constant<int, 64>{});
    }
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
