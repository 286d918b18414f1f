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
//   O^T[d][row]  += V^T[d][key] . P^T[key][row] (A = V^T tile from LDS, B = P in registers)
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
#include "tt_internal.h"

namespace tt {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr float kTau = 8.0f;  // lazy rescale threshold (log2 units)
constexpr float kLn2 = 0.693147180559945309f;

template <int D>
struct Cfg {
    static constexpr int KSTR = D + 8;        // K row stride in LDS (elements), 16-byte pad
    static constexpr int VSTR = kTile + 8;    // V^T row stride in LDS (elements)
    static constexpr int K_ELEMS = kTile * KSTR;
    static constexpr int V_ELEMS = D * VSTR;
    static constexpr int BUF = K_ELEMS + V_ELEMS;
    static constexpr int DS = D / 16;         // k-steps of the score product
    static constexpr int DT = D / 32;         // d tiles of the output product
    static constexpr int CHUNKS = D / 8;      // 16-byte chunks per K/V row
    static constexpr int KPT = kTile * CHUNKS / kThreads;  // keys per thread per tile
};

struct Args {
    const uint16_t* Q;
    long long qsb, qss, qsh;
    const uint16_t* Kc;
    const uint16_t* Vc;
    int page_size, num_pages, max_pages, Lmax;
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

__device__ __forceinline__ int seq_len(const Args& a, int b) {
    return a.ctx_len ? clamp_len(a.ctx_len[b], a.Lmax) : 0;
}
__device__ __forceinline__ int units_for(const Args& a, int L) { return (L + kTile - 1) / kTile + a.has_den; }

// Block-wide: total units W and, for unit u (u >= 0), the sequence holding it
// and the first unit of that sequence. For b_prefix >= 0 instead, also the
// first unit of sequence b_prefix. `sh` is LDS scratch of 260 ints.
__device__ void scan_units(const Args& a, int u, int b_prefix, int* sh, int& W, int& b_out, int& c_out) {
    const int t = threadIdx.x;
    const int mult = a.Hkv * a.n_rb;
    const int chunk = (a.B + kThreads - 1) / kThreads;
    const int lo = min(a.B, t * chunk), hi = min(a.B, lo + chunk);
    int sum = 0, before = 0;
    for (int b = lo; b < hi; ++b) {
        const int n = units_for(a, seq_len(a, b)) * mult;
        sum += n;
        if (b < b_prefix) before += n;
    }
    sh[t] = sum;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int v = t >= off ? sh[t - off] : 0;
        __syncthreads();
        sh[t] += v;
        __syncthreads();
    }
    const int incl = sh[t];
    const int excl = incl - sum;
    W = sh[kThreads - 1];
    __syncthreads();
    if (t == 0) { sh[256] = 0; sh[257] = 0; sh[258] = 0; }
    __syncthreads();
    if (u >= 0 && u >= excl && u < incl) {
        int c = excl;
        for (int b = lo; b < hi; ++b) {
            const int n = units_for(a, seq_len(a, b)) * mult;
            if (u < c + n) { sh[256] = b; sh[257] = c; break; }
            c += n;
        }
    }
    if (b_prefix >= 0 && b_prefix >= lo && b_prefix < hi) sh[258] = excl + before;
    else if (b_prefix >= 0 && b_prefix == a.B && t == kThreads - 1) sh[258] = incl;
    __syncthreads();
    if (u >= 0) { b_out = sh[256]; c_out = sh[257]; }
    if (b_prefix >= 0) c_out = sh[258];
    __syncthreads();
}

struct Cur {
    int b, pl, t;    // sequence, pair index within the sequence (g*n_rb + rb), tile within the pair
    int L, units;    // prefix length, tiles per pair of sequence b
};

__device__ __forceinline__ void advance(Cur& c, const Args& a) {
    if (++c.t < c.units) return;
    c.t = 0;
    if (++c.pl < a.Hkv * a.n_rb) return;
    c.pl = 0;
    for (;;) {
        if (++c.b >= a.B) { c.units = 1; return; }
        c.L = seq_len(a, c.b);
        c.units = units_for(a, c.L);
        if (c.units > 0) return;
    }
}

template <int D>
struct Regs {
    u32x4 k[Cfg<D>::KPT];
    u32x4 v[Cfg<D>::KPT];
};

__device__ __forceinline__ u32x4 ldg_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// global -> registers: this thread's KPT keys x one 16-byte chunk of the tile at c
template <int D>
__device__ __forceinline__ void load_tile(Regs<D>& r, const Cur& c, const Args& a) {
    using C = Cfg<D>;
    const int tid = threadIdx.x;
    const int kg = tid / C::CHUNKS, ch = tid % C::CHUNKS;
    const int g = c.pl / a.n_rb;
    const int nct = (c.L + kTile - 1) / kTile;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (c.t < nct) {
        const int j0 = c.t * kTile + kg * C::KPT;  // KPT consecutive keys, all in one page
        int page = -1;
        if (j0 < c.L) page = a.page_table[(long long)c.b * a.max_pages + j0 / a.page_size];
        const bool ok = page >= 0 && page < a.num_pages;
        const long long base = (((long long)(ok ? page : 0) * a.Hkv + g) * a.page_size + j0 % a.page_size) * D + ch * 8;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const bool valid = ok && (j0 + i < c.L);
            r.k[i] = valid ? ldg_nt(a.Kc + base + (long long)i * D) : z;
            r.v[i] = valid ? ldg_nt(a.Vc + base + (long long)i * D) : z;
        }
    } else {
        const long long base = (long long)c.b * a.dsb + (long long)g * a.dsh + ch * 8;
#pragma unroll
        for (int i = 0; i < C::KPT; ++i) {
            const int j = kg * C::KPT + i;
            const bool valid = j < a.S;
            r.k[i] = valid ? ldg_nt(a.Kd + base + (long long)j * a.dss) : z;
            r.v[i] = valid ? ldg_nt(a.Vd + base + (long long)j * a.dss) : z;
        }
    }
}

// position of key k inside a V^T row: within each 16-key group, bits 2 and 3
// of the key index are swapped, so the 8 keys one lane feeds to a 16-key
// MFMA step (keys 4h..4h+3 and 8+4h..8+4h+3, h = lane / 32) sit contiguously.
__device__ __forceinline__ int vpos(int k) {
    return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

template <int D>
__device__ __forceinline__ void store_tile(const Regs<D>& r, uint16_t* buf) {
    using C = Cfg<D>;
    const int tid = threadIdx.x;
    const int kg = tid / C::CHUNKS, ch = tid % C::CHUNKS;
    uint16_t* Ks = buf;
    uint16_t* Vt = buf + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i)
        *reinterpret_cast<u32x4*>(Ks + (kg * C::KPT + i) * C::KSTR + ch * 8) = r.k[i];
    const int pos = vpos(kg * C::KPT);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        unsigned w[C::KPT / 2];
#pragma unroll
        for (int i = 0; i < C::KPT / 2; ++i) {
            const unsigned lo = (r.v[2 * i][e >> 1] >> sh) & 0xffffu;
            const unsigned hi = (r.v[2 * i + 1][e >> 1] >> sh) & 0xffffu;
            w[i] = lo | (hi << 16);
        }
        uint16_t* dst = Vt + (ch * 8 + e) * C::VSTR + pos;
        if constexpr (C::KPT == 4) {
            u32x2 v2 = {w[0], w[1]};
            *reinterpret_cast<u32x2*>(dst) = v2;
        } else {
            *reinterpret_cast<unsigned*>(dst) = w[0];
        }
    }
}

__device__ __forceinline__ bf16x8 lds16(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_round(float x) {
    return (float)(__bf16)x;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(Args a) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];
    __shared__ int sh[260];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hl = lane >> 5;

    // logical segment of this workgroup: consecutive segments share an XCD
    const int per_xcd = a.n_seg / 8;
    const int seg = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;

    int W, b0, c0;
    // first pass: total units (needed for the segment length)
    scan_units(a, -1, -1, sh, W, b0, c0);
    const int seg_len = (W + a.n_seg - 1) / a.n_seg;
    const int u0 = seg * seg_len;
    const int u1 = min(W, u0 + seg_len);
    if (u0 >= u1) return;
    scan_units(a, u0, -1, sh, W, b0, c0);

    Cur nxt;
    nxt.b = b0;
    nxt.L = seq_len(a, b0);
    nxt.units = units_for(a, nxt.L);
    {
        const int off = u0 - c0;
        nxt.pl = off / nxt.units;
        nxt.t = off % nxt.units;
    }
    const int mult = a.Hkv * a.n_rb;

    Regs<D> regs;
    load_tile<D>(regs, nxt, a);

    bf16x8 qf[2][C::DS];
    f32x16 oacc[C::DT][2];
    float m2[2], lsum[2];
    int piece_t0 = 0;
    int buf = 0;

    for (int u = u0; u < u1; ++u) {
        uint16_t* B = smem + buf * C::BUF;
        store_tile<D>(regs, B);
        __syncthreads();
        const Cur c = nxt;
        if (u + 1 < u1) {
            advance(nxt, a);
            load_tile<D>(regs, nxt, a);
        }
        const int g = c.pl / a.n_rb, rb = c.pl % a.n_rb;
        if (u == u0 || c.t == 0) {
            // new piece: query rows of (b, g, rb), fresh softmax state
            piece_t0 = c.t;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int rr = rb * kRows + wave * 64 + nt * 32 + l32;
                const bool valid = rr < a.S * a.G;
                const int s = valid ? rr / a.G : 0, h = g * a.G + (valid ? rr % a.G : 0);
                const uint16_t* q = a.Q + c.b * a.qsb + s * a.qss + h * a.qsh + hl * 8;
#pragma unroll
                for (int ds = 0; ds < C::DS; ++ds) {
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    const u32x4 v = valid ? *reinterpret_cast<const u32x4*>(q + ds * 16) : z;
                    qf[nt][ds] = __builtin_bit_cast(bf16x8, v);
                }
                m2[nt] = -INFINITY;
                lsum[nt] = 0.f;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dt][nt][i] = 0.f;
            }
        }
        const int nct = (c.L + kTile - 1) / kTile;
        const int nvalid = c.t < nct ? min(kTile, c.L - c.t * kTile) : a.S;

        // ---- scores: S^T[key][row] for 64 keys x 64 rows of this wave ----
        const uint16_t* Ks = B;
        const uint16_t* Vt = B + C::K_ELEMS;
        f32x16 sacc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) sacc[mt][nt][i] = 0.f;
#pragma unroll
        for (int ds = 0; ds < C::DS; ++ds) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 kf = lds16(Ks + (mt * 32 + l32) * C::KSTR + ds * 16 + hl * 8);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    sacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[nt][ds], sacc[mt][nt], 0, 0, 0);
            }
        }
        if (nvalid < kTile) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = mt * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
                    if (key >= nvalid) {
                        sacc[mt][0][i] = -INFINITY;
                        sacc[mt][1][i] = -INFINITY;
                    }
                }
        }
        // ---- online softmax (exp2 domain) ----
        float mnew[2];
        bool need[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mt][nt][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            mnew[nt] = mx * a.c_log2;
            need[nt] = mnew[nt] > m2[nt] + kTau;
        }
        if (__any(need[0] || need[1])) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float alpha = 1.f;
                if (need[nt]) {
                    alpha = __builtin_amdgcn_exp2f(m2[nt] - mnew[nt]);
                    m2[nt] = mnew[nt];
                }
                lsum[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dt][nt][i] *= alpha;
            }
        }
        bf16x8 pf[4][2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const float neg = -m2[nt];
            float ls = 0.f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f32x8 pv;
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    pv[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[ks >> 1][nt][(ks & 1) * 8 + t], a.c_log2, neg));
                const bf16x8 pb = __builtin_convertvector(pv, bf16x8);
                pf[ks][nt] = pb;
#pragma unroll
                for (int t = 0; t < 8; ++t) ls += (float)pb[t];
            }
            lsum[nt] += ls;
        }
        // ---- O^T[d][row] += V^T . P^T ----
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int dt = 0; dt < C::DT; ++dt) {
                const bf16x8 vf = lds16(Vt + (dt * 32 + l32) * C::VSTR + ks * 16 + hl * 8);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks][nt], oacc[dt][nt], 0, 0, 0);
            }
        }

        // ---- end of piece: write the result or a partial ----
        if (c.t == c.units - 1 || u == u1 - 1) {
            const bool full = piece_t0 == 0 && c.t == c.units - 1;
            const int p = c.b * mult + c.pl;
            const int slot = seg + p;
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const float lt = lsum[nt] + __shfl_xor(lsum[nt], 32);
                const float inv = 1.f / lt;
                const float lse = (m2[nt] + __log2f(lt)) * kLn2;
                const int rl = wave * 64 + nt * 32 + l32;  // row within the block
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
                            f32x4 o = {oacc[dt][nt][j * 4] * inv, oacc[dt][nt][j * 4 + 1] * inv,
                                       oacc[dt][nt][j * 4 + 2] * inv, oacc[dt][nt][j * 4 + 3] * inv};
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
                            f32x4 o = {oacc[dt][nt][j * 4] * inv, oacc[dt][nt][j * 4 + 1] * inv,
                                       oacc[dt][nt][j * 4 + 2] * inv, oacc[dt][nt][j * 4 + 3] * inv};
                            *reinterpret_cast<f32x4*>(po + d) = o;
                        }
                    if (hl == 0) a.part_lse[(long long)slot * kRows + rl] = lse;
                }
            }
        }
        buf ^= 1;
    }
}

// Merge the per-segment partials of every pair that segment boundaries cut,
// and write O = 0, LSE = -inf for pairs with no keys at all.
// Grid: n_pairs * 16 workgroups of 256 threads, 16 rows each.
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bf16_finalize(Args a) {
    __shared__ int sh[260];
    const int mult = a.Hkv * a.n_rb;
    const int p = blockIdx.x / 16, chunk = blockIdx.x % 16;
    const int b = p / mult, pl = p % mult;
    const int g = pl / a.n_rb, rb = pl % a.n_rb;
    int W, bdummy, Cb;
    scan_units(a, -1, b, sh, W, bdummy, Cb);
    const int units = units_for(a, seq_len(a, b));
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
    if (p.head_dim == 128) {
        hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(pl.n_seg), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(attn_bf16_finalize<128>, dim3(pl.n_pairs * 16), dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(pl.n_seg), dim3(kThreads), 0, s, a);
        hipLaunchKernelGGL(attn_bf16_finalize<64>, dim3(pl.n_pairs * 16), dim3(kThreads), 0, s, a);
    }
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
