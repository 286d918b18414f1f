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
// tiles of all pairs are laid end to end and cut into equal segments, one
// per workgroup, so every CU streams the same number of tiles whatever the
// spread of prefix lengths. A pair that lies inside one segment is written
// directly; a pair cut by segment boundaries leaves one fp32 partial
// (O normalised, LSE) per segment, merged by a second kernel. Segments are
// numbered so that consecutive ones run on the same XCD, which keeps a pair's
// partials in one L2.
#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#ifndef TT_ATTN_WAVES
#define TT_ATTN_WAVES 8
#endif
#ifndef TT_ATTN_PREFETCH
#define TT_ATTN_PREFETCH 2
#endif
constexpr int kWaves = TT_ATTN_WAVES;       // waves per workgroup; each owns kRows / kWaves query rows
constexpr int kNT = kRows / (32 * kWaves);  // 32-row MFMA tiles per wave
constexpr int kNR = TT_ATTN_PREFETCH;       // tiles in flight in registers (1 or 2)
static_assert(kNT >= 1 && kNR >= 1 && kNR <= 2, "unsupported attention kernel shape");
constexpr int kThreads = 64 * kWaves;
constexpr int kFinThreads = 256;
constexpr float kTau = 8.0f;  // lazy rescale threshold (log2 units)
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Cfg {
    static constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
    static constexpr int ROWB = D * 2;             // bytes per row (rows are not padded)
    static constexpr int TILEB = kTile * ROWB;     // bytes of one K (or V) tile
    static constexpr int STAGEB = 2 * TILEB;       // K then V
    static constexpr int LPK = kTile * CPR / kThreads;  // 16-byte K (and V) loads per thread per tile
    static constexpr int DS = D / 16;              // k-steps of the score product
    static constexpr int DT = D / 32;              // d tiles of the output product
    static_assert(LPK >= 1 && LPK <= 4, "up to four chunks of K and of V per thread and tile");
};

// Rows sit unpadded in LDS; the 16-byte chunk c of row r is stored at chunk
// position c ^ swz(r). Over any 16 consecutive rows (the rows one 16-lane
// phase of a K-operand read touches) and over the 4-row x 4-chunk blocks of a
// transposing V read, the swizzle sends the accessed chunks to distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

struct Args {
    const uint16_t* Q;
    long long qsb, qss, qsh;
    const uint16_t* Kc;
    const uint16_t* Vc;
    int page_size, num_pages, max_pages, Lmax;
    int page_shift;  // log2(page_size) when it is a power of two
    const int* page_table;
    const int* ctx_len;
    const uint16_t* Kd;
    const uint16_t* Vd;
    long long dsb, dss, dsh;
    void* O;
    long long osb, oss, osh;
    int o_f32;
    float* LSE;
    float* part_o;
    float* part_lse;
    int B, S, Hq, Hkv, G, n_rb, has_den, n_seg;
    float c_log2;  // softmax_scale * log2(e)
};

__device__ __forceinline__ int seq_len(const Args& a, const int* __restrict__ ctx_len, int b) {
    return ctx_len ? clamp_len(ctx_len[b], a.Lmax) : 0;
}
__device__ __forceinline__ int units_for(const Args& a, int L) { return (L + kTile - 1) / kTile + a.has_den; }

// Block-wide: total units W and, for unit u (u >= 0), the sequence holding it
// and the first unit of that sequence. For b_prefix >= 0 instead, also the
// first unit of sequence b_prefix. `sh` is LDS scratch of NTHR + 4 ints.
template <int NTHR>
__device__ void scan_units(const Args& a, const int* __restrict__ ctx_len, int u, int b_prefix, int* sh, int& W,
                           int& b_out, int& c_out) {
    const int t = threadIdx.x;
    const int mult = a.Hkv * a.n_rb;
    const int chunk = (a.B + NTHR - 1) / NTHR;
    const int lo = min(a.B, t * chunk), hi = min(a.B, lo + chunk);
    int sum = 0, before = 0;
    for (int b = lo; b < hi; ++b) {
        const int n = units_for(a, seq_len(a, ctx_len, b)) * mult;
        sum += n;
        if (b < b_prefix) before += n;
    }
    sh[t] = sum;
    __syncthreads();
    for (int off = 1; off < NTHR; off <<= 1) {
        const int v = t >= off ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += v;
        __syncthreads();
    }
    const int incl = sh[t];
    const int excl = incl - sum;
    W = sh[NTHR - 1];
    __syncthreads();
    if (t == 0) { sh[NTHR] = 0; sh[NTHR + 1] = 0; sh[NTHR + 2] = 0; }
    __syncthreads();
    if (u >= 0 && u >= excl && u < incl) {
        int c = excl;
        for (int b = lo; b < hi; ++b) {
            const int n = units_for(a, seq_len(a, ctx_len, b)) * mult;
            if (u < c + n) { sh[NTHR] = b; sh[NTHR + 1] = c; break; }
            c += n;
        }
    }
    if (b_prefix >= 0 && b_prefix >= lo && b_prefix < hi) sh[NTHR + 2] = excl + before;
    else if (b_prefix >= 0 && b_prefix == a.B && t == NTHR - 1) sh[NTHR + 2] = incl;
    __syncthreads();
    if (u >= 0) { b_out = sh[NTHR]; c_out = sh[NTHR + 1]; }
    if (b_prefix >= 0) c_out = sh[NTHR + 2];
    __syncthreads();
}

struct Cur {
    int b, pl, t;    // sequence, pair index within the sequence (g*n_rb + rb), tile within the pair
    int L, units;    // prefix length, tiles per pair of sequence b
    int nct;         // prefix tiles of sequence b
    int g, rb;       // kv head and row block of pair pl
};

__device__ __forceinline__ void set_seq(Cur& c, const Args& a, const int* __restrict__ ctx_len, int b) {
    c.b = b;
    c.L = seq_len(a, ctx_len, b);
    c.nct = (c.L + kTile - 1) / kTile;
    c.units = c.nct + a.has_den;
}

__device__ __forceinline__ void set_pair(Cur& c, const Args& a, int pl) {
    c.pl = pl;
    c.g = pl / a.n_rb;
    c.rb = pl - c.g * a.n_rb;
}

__device__ __forceinline__ void advance(Cur& c, const Args& a, const int* __restrict__ ctx_len) {
    if (++c.t < c.units) return;
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

__device__ __forceinline__ u32x4 ldg_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---- tile loads: global -> registers -> LDS --------------------------------
// Thread t moves chunk (t + kThreads*i) of each tile: row r = that / CPR, 16-byte
// chunk c = that % CPR. The rows a wave touches for one i lie in one 16-aligned
// group of keys, hence in one page, so the page id is wave-uniform (a scalar
// load, issued one tile ahead of the loads that use it).
template <int D>
struct Regs {
    u32x4 k[Cfg<D>::LPK];
    u32x4 v[Cfg<D>::LPK];
};

struct Pages {
    int p[4];
};

template <int D, bool P2>
__device__ __forceinline__ Pages tile_pages(const Cur& c, const Args& a, const int* __restrict__ page_table) {
    using C = Cfg<D>;
    Pages pg{{0, 0, 0, 0}};
    if (c.t >= c.nct) return pg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int i = 0; i < C::LPK; ++i) {
        const int r = (wave * 64 + kThreads * i) / C::CPR;  // first row of this wave's block
        const int j0 = min(c.t * kTile + r, c.L - 1);
        pg.p[i] = page_table[(long long)c.b * a.max_pages + page_of<P2>(a, j0)];
    }
    return pg;
}

// Issue this thread's loads of the tile at c. Loads are unconditional and their
// registers are not touched until they are stored to LDS: a key past the end of
// a partial tile reads the tile's last valid key instead (finite, weight exactly
// 0); a page id outside [0, num_pages) is clamped, so a corrupt table reads
// wrong data but never faults.
template <int D, bool P2>
__device__ __forceinline__ void load_tile(Regs<D>& r, const Cur& c, const Pages& pg, const Args& a) {
    using C = Cfg<D>;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ch = lane % C::CPR;       // 16-byte chunk of the row (64 is a multiple of CPR)
    const int lrow = lane / C::CPR;     // row offset within this wave's block
#pragma unroll
    for (int i = 0; i < C::LPK; ++i) {
        const int rbase = (wave * 64 + kThreads * i) / C::CPR;  // uniform first row of the block
        // wave-uniform base pointer plus a 32-bit per-lane element offset
        const uint16_t* kb;
        const uint16_t* vb;
        unsigned off;
        if (c.t < c.nct) {
            const int page = min(max(pg.p[i], 0), a.num_pages - 1);
            const long long pbase = ((long long)page * a.Hkv + c.g) * a.page_size * D;
            kb = a.Kc + pbase;
            vb = a.Vc + pbase;
            const int j = min(c.t * kTile + rbase + lrow, c.L - 1);
            off = (unsigned)(slot_of<P2>(a, j) * D + ch * 8);
        } else {
            const long long dbase = (long long)c.b * a.dsb + (long long)c.g * a.dsh;
            kb = a.Kd + dbase;
            vb = a.Vd + dbase;
            off = (unsigned)(min(rbase + lrow, a.S - 1) * (int)a.dss + ch * 8);
        }
        r.k[i] = ldg_nt(kb + off);
        r.v[i] = ldg_nt(vb + off);
    }
}

// registers -> LDS stage, chunk c of row r at chunk position c ^ swz(r)
template <int D>
__device__ __forceinline__ void store_tile(const Regs<D>& r, uint8_t* stage) {
    using C = Cfg<D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < C::LPK; ++i) {
        const int q = tid + kThreads * i;
        const int row = q / C::CPR, ch = q % C::CPR;
        const int off = row * C::ROWB + 16 * (ch ^ swz<D>(row));
        *reinterpret_cast<u32x4*>(stage + off) = r.k[i];
        *reinterpret_cast<u32x4*>(stage + C::TILEB + off) = r.v[i];
    }
}

// Workgroup barrier ordering LDS accesses only: waits for this wave's own LDS
// writes, not for the global loads in flight (a plain __syncthreads() would
// wait for those too and drain the prefetch).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bf16x8 lds16(const uint8_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element i%4 of the 8-byte rows read by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ i16x4 lds_tr(const uint8_t* p) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// Per-wave state carried across tiles.
template <int D>
struct State {
    bf16x8 qf[kNT][Cfg<D>::DS];
    f32x16 oacc[Cfg<D>::DT][kNT];
    f32x16 lacc[kNT];  // row sums of the rounded weights, from an MFMA against ones
    float m2[kNT];
    int piece_t0;
};

template <int D, bool P2>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(Args a, const int* __restrict__ page_table,
                                                                const int* __restrict__ ctx_len) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGEB];
    __shared__ int sh[kThreads + 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    // logical segment of this workgroup: consecutive segments share an XCD
    const int per_xcd = a.n_seg / 8;
    const int seg = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;

    int W, b0, c0;
    scan_units<kThreads>(a, ctx_len, -1, -1, sh, W, b0, c0);  // total units W
    W = __builtin_amdgcn_readfirstlane(W);                     // uniform: keep the walk in scalar registers
    const int seg_len = (W + a.n_seg - 1) / a.n_seg;
    const int u0 = seg * seg_len;
    const int u1 = min(W, u0 + seg_len);
    if (u0 >= u1) return;
    scan_units<kThreads>(a, ctx_len, u0, -1, sh, W, b0, c0);
    b0 = __builtin_amdgcn_readfirstlane(b0);
    c0 = __builtin_amdgcn_readfirstlane(c0);

    Cur cc;  // tile being computed
    set_seq(cc, a, ctx_len, b0);
    {
        const int off = u0 - c0;
        set_pair(cc, a, off / cc.units);
        cc.t = off % cc.units;
    }
    const int mult = a.Hkv * a.n_rb;

    // kNR register sets carry tiles u+1 .. u+kNR while tile u is computed: a tile's
    // loads are issued kNR iterations before its registers are stored to LDS.
    Regs<D> R[kNR];
    Cur cl = cc;  // next tile to load
    int ul = u0;
    Pages pg = tile_pages<D, P2>(cl, a, page_table);
#pragma unroll
    for (int k = 0; k < kNR; ++k) {
        if (ul < u1) {
            load_tile<D, P2>(R[k], cl, pg, a);
            if (++ul < u1) {
                advance(cl, a, ctx_len);
                pg = tile_pages<D, P2>(cl, a, page_table);
            }
        }
    }
    bf16x8 ones;
#pragma unroll
    for (int t = 0; t < 8; ++t) ones[t] = (__bf16)1.0f;

    State<D> st;
    st.piece_t0 = 0;
    // lane-constant parts of the swizzled LDS addresses
    const int ksw = swz<D>(l32);
    const int vrow = 4 * hl + ((lane & 15) >> 2);
    const int vsw0 = swz<D>(vrow), vsw1 = swz<D>(vrow + 8);
    const int vchunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int vbyte = 8 * (lane & 1);

    // one tile; S is the register set / LDS stage of tile u (u - u0 even: 0)
    auto step = [&](auto S_, int u) __attribute__((always_inline)) {
        constexpr int S = decltype(S_)::value;
        uint8_t* stage = smem + S * C::STAGEB;
        store_tile<D>(R[S % kNR], stage);
        lds_barrier();
        const Cur c = cc;
        const int g = c.g, rb = c.rb;
        const bool new_piece = u == u0 || c.t == 0;
        if (new_piece) {
            // query rows of (b, g, rb), in registers for the whole piece; issued
            // before the next loads so that waiting for them leaves those in flight
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const int rr = rb * kRows + (wave * kNT + nt) * 32 + l32;
                const bool valid = rr < a.S * a.G;
                const int s = valid ? rr / a.G : 0, h = g * a.G + (valid ? rr % a.G : 0);
                const uint16_t* q = a.Q + c.b * a.qsb + s * a.qss + h * a.qsh + hl * 8;
#pragma unroll
                for (int ds = 0; ds < C::DS; ++ds) {
                    u32x4 v = *reinterpret_cast<const u32x4*>(q + ds * 16);
                    if (!valid) v = u32x4{0u, 0u, 0u, 0u};
                    st.qf[nt][ds] = __builtin_bit_cast(bf16x8, v);
                }
            }
        }
        // refill this register set with tile u + kNR
        if (ul < u1) {
            load_tile<D, P2>(R[S % kNR], cl, pg, a);
            if (++ul < u1) {
                advance(cl, a, ctx_len);
                pg = tile_pages<D, P2>(cl, a, page_table);
            }
        }
        if (new_piece) {
            st.piece_t0 = c.t;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                st.m2[nt] = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) st.lacc[nt][i] = 0.f;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) st.oacc[dt][nt][i] = 0.f;
            }
        }
        const int nvalid = c.t < c.nct ? min(kTile, c.L - c.t * kTile) : a.S;
        const uint8_t* Kst = stage;
        const uint8_t* Vst = stage + C::TILEB;

        // ---- scores: S^T[key][row] for 64 keys x 32*kNT rows of this wave ----
        f32x16 sacc[2][kNT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[mt][nt][i] = 0.f;
        // the two 32-key halves accumulate in alternation: independent MFMA chains
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
            bf16x8 kf[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
                kf[mt] = lds16(Kst + (mt * 32 + l32) * C::ROWB + 16 * ((2 * ds + hl) ^ ksw));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
                    sacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[mt], st.qf[nt][ds], sacc[mt][nt], 0, 0, 0);
            if (ds & 1) __builtin_amdgcn_sched_barrier(0);  // bound how far reads run ahead
        }
        if (nvalid < kTile) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = mt * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
                    if (key >= nvalid) {
#pragma unroll
                        for (int nt = 0; nt < kNT; ++nt) sacc[mt][nt][i] = -INFINITY;
                    }
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- online softmax (exp2 domain) ----
        float mnew[kNT];
        bool need[kNT];
        bool any_need = false;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mt][nt][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mnew[nt] = mx * a.c_log2;
            need[nt] = mnew[nt] > st.m2[nt] + kTau;
            any_need = any_need || need[nt];
        }
        if (__any(any_need)) {
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                float alpha = 1.f;
                if (need[nt]) {
                    alpha = __builtin_amdgcn_exp2f(st.m2[nt] - mnew[nt]);
                    st.m2[nt] = mnew[nt];
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) st.lacc[nt][i] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) st.oacc[dt][nt][i] *= alpha;
            }
        }
        bf16x8 pf[4][kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
            const float neg = -st.m2[nt];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f32x8 pv;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    pv[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ks >> 1][nt][(ks & 1) * 8 + t], a.c_log2, neg));
                pf[ks][nt] = __builtin_convertvector(pv, bf16x8);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- O^T[d][row] += V^T . P^T ----
        // V sits in LDS as [key][d]; the transposing read hands lane l the four keys
        // kb..kb+3 of column d = 32*dt + l%32, with kb = 16*ks + 8*half + 4*(l/32):
        // exactly the keys its P^T slots hold.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 vf[C::DT];
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const int cv = 4 * dt + vchunk;
                const uint8_t* p0 = Vst + (ks * 16 + vrow) * C::ROWB + 16 * (cv ^ vsw0) + vbyte;
                const uint8_t* p1 = Vst + (ks * 16 + vrow + 8) * C::ROWB + 16 * (cv ^ vsw1) + vbyte;
                const i16x4 pair[2] = {lds_tr(p0), lds_tr(p1)};
                vf[dt] = __builtin_bit_cast(bf16x8, pair);
            }
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                for (int nt = 0; nt < kNT; ++nt)
                    st.oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt], pf[ks][nt], st.oacc[dt][nt], 0, 0, 0);
            // every row of ones . P^T is the row sum over these 16 keys
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
                st.lacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf[ks][nt], st.lacc[nt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- end of piece: write the result or a partial ----
        if (c.t == c.units - 1 || u == u1 - 1) {
            const bool full = st.piece_t0 == 0 && c.t == c.units - 1;
            const int p = c.b * mult + c.pl;
            const int slot = seg + p;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt) {
                const float lt = st.lacc[nt][0];
                const float inv = 1.f / lt;
                const float lse = (st.m2[nt] + __log2f(lt)) * kLn2;
                const int rl = (wave * kNT + nt) * 32 + l32;  // row within the block
                const int rr = rb * kRows + rl;
                if (rr >= a.S * a.G) continue;
                if (full) {
                    const int s = rr / a.G, h = g * a.G + rr % a.G;
                    const long long ob = c.b * a.osb + s * a.oss + h * a.osh;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int d = dt * 32 + j * 8 + hl * 4;
                            f32x4 o = {st.oacc[dt][nt][j * 4] * inv, st.oacc[dt][nt][j * 4 + 1] * inv,
                                       st.oacc[dt][nt][j * 4 + 2] * inv, st.oacc[dt][nt][j * 4 + 3] * inv};
                            if (a.o_f32) {
                                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.O) + ob + d) = o;
                            } else {
                                typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                                const bf16x4 ob4 = __builtin_convertvector(o, bf16x4);
                                *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.O) + ob + d) = ob4;
                            }
                        }
                    if (a.LSE && hl == 0) a.LSE[((long long)c.b * a.Hq + h) * a.S + s] = lse;
                } else {
                    float* po = a.part_o + ((long long)slot * kRows + rl) * D;
#pragma unroll
                    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int d = dt * 32 + j * 8 + hl * 4;
                            f32x4 o = {st.oacc[dt][nt][j * 4] * inv, st.oacc[dt][nt][j * 4 + 1] * inv,
                                       st.oacc[dt][nt][j * 4 + 2] * inv, st.oacc[dt][nt][j * 4 + 3] * inv};
                            *reinterpret_cast<f32x4*>(po + d) = o;
                        }
                    if (hl == 0) a.part_lse[(long long)slot * kRows + rl] = lse;
                }
            }
        }
        if (u + 1 < u1) advance(cc, a, ctx_len);
    };

    for (int u = u0; u < u1; u += 2) {
        step(std::integral_constant<int, 0>{}, u);
        if (u + 1 < u1) step(std::integral_constant<int, 1>{}, u + 1);
    }
}

// Merge the per-segment partials of every pair that segment boundaries cut,
// and write O = 0, LSE = -inf for pairs with no keys at all.
// Grid: n_pairs * 16 workgroups of 256 threads, 16 rows each.
template <int D>
__global__ __launch_bounds__(kFinThreads) void attn_bf16_finalize(Args a, const int* __restrict__ ctx_len) {
    __shared__ int sh[kFinThreads + 4];
    const int mult = a.Hkv * a.n_rb;
    const int p = blockIdx.x / 16, chunk = blockIdx.x % 16;
    const int b = p / mult, pl = p % mult;
    const int g = pl / a.n_rb, rb = pl % a.n_rb;
    int W, bdummy, Cb;
    scan_units<kFinThreads>(a, ctx_len, -1, b, sh, W, bdummy, Cb);
    const int units = units_for(a, seq_len(a, ctx_len, b));  // tiles per pair
    const int seg_len = (W + a.n_seg - 1) / a.n_seg;
    int s0 = 0, s1 = -1;
    if (units > 0) {
        const int U = Cb + pl * units;
        s0 = U / seg_len;
        s1 = (U + units - 1) / seg_len;
        if (s0 == s1) return;  // written by the main kernel
    }
    const int tid = threadIdx.x;
    const int rl = chunk * 16 + tid / 16;      // row within the block
    const int rr = rb * kRows + rl;
    if (rr >= a.S * a.G) return;
    const int s = rr / a.G, h = g * a.G + rr % a.G;
    const long long ob = b * a.osb + s * a.oss + h * a.osh;
    float M = -INFINITY;
    for (int sg = s0; sg <= s1; ++sg) M = fmaxf(M, a.part_lse[(long long)(sg + p) * kRows + rl]);
    constexpr int PER = D / 64;  // 4-float chunks per thread
    f32x4 acc[PER];
    for (int k = 0; k < PER; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    float Wsum = 0.f;
    if (M != -INFINITY) {
        for (int sg = s0; sg <= s1; ++sg) {
            const long long slot = sg + p;
            const float l = a.part_lse[slot * kRows + rl];
            if (l == -INFINITY) continue;
            const float w = __expf(l - M);
            Wsum += w;
            const float* po = a.part_o + (slot * kRows + rl) * D;
            for (int k = 0; k < PER; ++k) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(po + ((tid % 16) + 16 * k) * 4);
                acc[k] += w * v;
            }
        }
    }
    const float inv = Wsum > 0.f ? 1.f / Wsum : 0.f;
    for (int k = 0; k < PER; ++k) {
        const int d = ((tid % 16) + 16 * k) * 4;
        const f32x4 o = acc[k] * inv;
        if (a.o_f32) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.O) + ob + d) = o;
        } else {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(a.O) + ob + d) = __builtin_convertvector(o, bf16x4);
        }
    }
    if (a.LSE && tid % 16 == 0)
        a.LSE[((long long)b * a.Hq + h) * a.S + s] = Wsum > 0.f ? M + __logf(Wsum) : -INFINITY;
}

}  // namespace

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
    pl.ws_part_o = (size_t)pl.n_slots * kRows * p.head_dim * sizeof(float);
    pl.ws_part_lse = (size_t)pl.n_slots * kRows * sizeof(float);
    pl.ws_total = pl.ws_part_o + pl.ws_part_lse + 256;
    return pl;
}

tt_status launch_attn_bf16(const tt_block_attn_params& p, const AttnPlan& pl, void* ws, hipStream_t s) {
    Args a{};
    a.Q = static_cast<const uint16_t*>(p.Q);
    a.qsb = p.q_stride_b; a.qss = p.q_stride_s; a.qsh = p.q_stride_h;
    a.Kc = static_cast<const uint16_t*>(p.Kctx);
    a.Vc = static_cast<const uint16_t*>(p.Vctx);
    a.page_size = p.page_size; a.num_pages = p.num_pages; a.max_pages = p.max_pages;
    const long long cap = (long long)p.max_pages * p.page_size;
    a.Lmax = (int)(p.max_ctx_len < cap ? p.max_ctx_len : cap);
    a.page_table = p.page_table;
    a.ctx_len = p.max_ctx_len > 0 ? p.ctx_len : nullptr;
    a.Kd = static_cast<const uint16_t*>(p.Kden);
    a.Vd = static_cast<const uint16_t*>(p.Vden);
    a.dsb = p.den_stride_b; a.dss = p.den_stride_s; a.dsh = p.den_stride_h;
    a.O = p.O;
    a.osb = p.o_stride_b; a.oss = p.o_stride_s; a.osh = p.o_stride_h;
    a.o_f32 = p.o_dtype == TT_F32;
    a.LSE = p.LSE;
    char* w = static_cast<char*>(ws);
    a.part_o = reinterpret_cast<float*>(w);
    a.part_lse = reinterpret_cast<float*>(w + pl.ws_part_o);
    a.B = p.B; a.S = p.S; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.Hq / p.Hkv;
    a.n_rb = pl.n_rb;
    a.has_den = p.Kden ? 1 : 0;
    a.n_seg = pl.n_seg;
    a.c_log2 = p.softmax_scale * 1.44269504088896340736f;
    a.page_shift = -1;
    if (p.page_size > 0 && (p.page_size & (p.page_size - 1)) == 0) {
        a.page_shift = 0;
        while ((1 << a.page_shift) < p.page_size) ++a.page_shift;
    }
    const bool p2 = a.page_shift >= 0;
    const dim3 grid(pl.n_seg), blk(kThreads), fgrid(pl.n_pairs * 16), fblk(kFinThreads);
    if (p.head_dim == 128) {
        if (p2) hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        else hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        hipLaunchKernelGGL(attn_bf16_finalize<128>, fgrid, fblk, 0, s, a, a.ctx_len);
    } else {
        if (p2) hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        else hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, blk, 0, s, a, a.page_table, a.ctx_len);
        hipLaunchKernelGGL(attn_bf16_finalize<64>, fgrid, fblk, 0, s, a, a.ctx_len);
    }
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
