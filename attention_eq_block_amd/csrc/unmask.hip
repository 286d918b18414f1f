// ConfidenceSample (Nemotron-TwoTower, arXiv 2606.26493, section 2.2
// "Sampling", Algorithm 2): one step of confidence unmasking.
//
// Kernel 1 (vocab_reduce): one pass over the logits of every MASKED row
// (unmasked rows are never read), gridded over rows x vocabulary splits. Each
// thread streams 16-byte chunks and keeps (max, first index of the max,
// sum of exp2((x - max) * log2(e)/temperature)); triples merge exactly across
// threads and splits, ties at the max going to the lower index.
// Kernel 2 (unmask_select): one wavefront per sequence, one lane per block
// position: confidence = 1/sum, then the commit rule -- every position above
// gamma if there are at least ceil(M/steps_left) of them, else the
// ceil(M/steps_left) most confident (ties to the lower position).
// Stochastic variant (the sampler's temperature argument, section 2.2
// "Sampling"), kernel 1b (sample_locate): a row with uniform u draws from
// softmax(x / temperature) by inverse transform sampling. The split masses of
// kernel 1 locate the split in which the cumulative sum passes u * Z; one
// workgroup re-reads only that split in iterations of 64 consecutive chunks,
// a scan of the iteration totals names the iteration where the sum passes, a
// scan of its chunk sums names the lane, and that lane walks its chunk to the
// first element whose cumulative sum passes. The drawn token's probability
// replaces the greedy confidence in kernel 2.
// The masked-diffusion loss L_MD (Eq. (4)) runs vocab_reduce at temperature 1
// and a one-workgroup finish (nll_finish): lse - x[target] per masked row and
// their mean.
#include <limits.h>

#include <type_traits>

#include "tt_internal.h"

namespace tt {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Triple {
    float m;
    int a;
    float z;
    float pad;
};

struct Drawn {
    int a;
    float conf;
};

struct UArgs {
    const void* logits;
    long long stride;
    const uint8_t* mask_in;
    uint8_t* mask_out;
    int* tokens;
    float* conf;
    int* num_masked;
    Triple* part;  // [n_vsplit][B*S]
    const float* uniforms;  // [B*S] or null (greedy)
    Drawn* drawn;           // [B*S] when sampling
    int B, S, V, n_vsplit, steps_left;
    float gamma, c;  // c = log2(e) / temperature
};

__device__ __forceinline__ void combine(float& m, int& a, float& z, float m2, int a2, float z2, float c) {
    const float M = fmaxf(m, m2);
    float zz = 0.f;
    if (M != -INFINITY) {
        if (m != -INFINITY) zz += z * __builtin_amdgcn_exp2f((m - M) * c);
        if (m2 != -INFINITY) zz += z2 * __builtin_amdgcn_exp2f((m2 - M) * c);
    }
    a = m > m2 ? a : (m2 > m ? a2 : min(a, a2));
    m = M;
    z = zz;
}

// fold 8 consecutive logits starting at index v into (m, a, z)
__device__ __forceinline__ void fold8(const float (&x)[8], int v, float& m, int& a, float& z, float c) {
    float cm = x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) cm = fmaxf(cm, x[k]);
    if (cm > m) {
        if (m != -INFINITY) z *= __builtin_amdgcn_exp2f((m - cm) * c);
        int k = 7;
#pragma unroll
        for (int kk = 7; kk >= 0; --kk) if (x[kk] == cm) k = kk;
        a = v + k;
        m = cm;
    }
    if (m != -INFINITY) {
        const float mc = m * c;
#pragma unroll
        for (int k = 0; k < 8; ++k) z += __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], c, -mc));
    }
}

__device__ __forceinline__ void unpack(const u32x4& r, float (&x)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(r[k] << 16);
        x[2 * k + 1] = __uint_as_float(r[k] & 0xffff0000u);
    }
}

// Element k of a row, widened to float.
template <bool BF16>
__device__ __forceinline__ float elem(const void* row, int k) {
    if (BF16) return __uint_as_float((unsigned)static_cast<const uint16_t*>(row)[k] << 16);
    return static_cast<const float*>(row)[k];
}

// Fold elements [lo, hi) (hi - lo <= 8) of a row as one padded chunk.
template <bool BF16>
__device__ __forceinline__ void fold_scalar(const void* row, int lo, int hi, float& m, int& a, float& z, float c) {
    float f[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] = lo + k < hi ? elem<BF16>(row, lo + k) : -INFINITY;
    fold8(f, lo, m, a, z, c);
}

// A row is cut as: a head of a0 < 8 elements up to the first 16-byte boundary,
// nfull aligned chunks of 8 elements, and a tail of fewer than 8. Split k of the
// grid takes an equal share of the chunks; split 0 also takes the head and the
// last split the tail. Each thread visits its elements in increasing index
// order, so the strict max update keeps the lowest index among its ties.
template <bool BF16>
__global__ __launch_bounds__(256) void vocab_reduce(UArgs a) {
    const int row = blockIdx.x;
    const int split = blockIdx.y;
    if (!a.mask_in[row]) return;
    constexpr int ES = BF16 ? 2 : 4;
    const char* rp = static_cast<const char*>(a.logits) + (long long)row * a.stride * ES;
    int a0 = (int)(((16u - (unsigned)(reinterpret_cast<uintptr_t>(rp) & 15u)) & 15u) / ES);
    if (a0 > a.V) a0 = a.V;
    const int nfull = (a.V - a0) / 8;
    const int per = (nfull + a.n_vsplit - 1) / a.n_vsplit;
    const int c0 = min(nfull, split * per), c1 = min(nfull, c0 + per);
    float m = -INFINITY, z = 0.f;
    int am = INT_MAX;
    const float c = a.c;
    if (split == 0 && threadIdx.x == 0 && a0 > 0) fold_scalar<BF16>(rp, 0, a0, m, am, z, c);
    const char* body = rp + a0 * ES;  // 16-byte aligned
    int ch = c0 + threadIdx.x;
    if (BF16) {
        for (; ch + 3 * 256 < c1; ch += 4 * 256) {
            u32x4 r[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + (ch + k * 256) * 16));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float f[8];
                unpack(r[k], f);
                fold8(f, a0 + (ch + k * 256) * 8, m, am, z, c);
            }
        }
        for (; ch < c1; ch += 256) {
            const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + ch * 16));
            float f[8];
            unpack(r, f);
            fold8(f, a0 + ch * 8, m, am, z, c);
        }
    } else {
        for (; ch + 256 < c1; ch += 2 * 256) {
            u32x4 r[4];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                r[2 * k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + (ch + k * 256) * 32));
                r[2 * k + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + (ch + k * 256) * 32 + 16));
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                float f[8];
                for (int e = 0; e < 4; ++e) { f[e] = __uint_as_float(r[2 * k][e]); f[4 + e] = __uint_as_float(r[2 * k + 1][e]); }
                fold8(f, a0 + (ch + k * 256) * 8, m, am, z, c);
            }
        }
        for (; ch < c1; ch += 256) {
            const u32x4 r0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + ch * 32));
            const u32x4 r1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(body + ch * 32 + 16));
            float f[8];
            for (int e = 0; e < 4; ++e) { f[e] = __uint_as_float(r0[e]); f[4 + e] = __uint_as_float(r1[e]); }
            fold8(f, a0 + ch * 8, m, am, z, c);
        }
    }
    const int t0 = a0 + nfull * 8;
    if (split == a.n_vsplit - 1 && threadIdx.x == 0 && t0 < a.V) fold_scalar<BF16>(rp, t0, a.V, m, am, z, c);
    // block reduction: wavefront shuffles, then across the 4 wavefronts
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off);
        const int a2 = __shfl_xor(am, off);
        const float z2 = __shfl_xor(z, off);
        combine(m, am, z, m2, a2, z2, c);
    }
    __shared__ Triple sh[4];
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = Triple{m, am, z, 0.f};
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < 4; ++k) combine(m, am, z, sh[k].m, sh[k].a, sh[k].z, c);
        a.part[(long long)split * a.B * a.S + row] = Triple{m, am, z, 0.f};
    }
}

// The raw bytes of 16-byte-aligned chunk ch of a row body (8 logits: r0, and
// r1 too for float32 logits), and the same widened to float.
template <bool BF16>
__device__ __forceinline__ void load_raw(const char* body, int ch, u32x4& r0, u32x4& r1) {
    if (BF16) {
        r0 = *reinterpret_cast<const u32x4*>(body + (long long)ch * 16);
    } else {
        r0 = *reinterpret_cast<const u32x4*>(body + (long long)ch * 32);
        r1 = *reinterpret_cast<const u32x4*>(body + (long long)ch * 32 + 16);
    }
}
template <bool BF16>
__device__ __forceinline__ void widen(const u32x4& r0, const u32x4& r1, float (&f)[8]) {
    if (BF16) {
        unpack(r0, f);
    } else {
        for (int e = 0; e < 4; ++e) { f[e] = __uint_as_float(r0[e]); f[4 + e] = __uint_as_float(r1[e]); }
    }
}
template <bool BF16>
__device__ __forceinline__ void load_chunk(const char* body, int ch, float (&f)[8]) {
    u32x4 r0, r1;
    load_raw<BF16>(body, ch, r0, r1);
    widen<BF16>(r0, r1, f);
}

// x of another lane by a DPP pattern (0 where the pattern names none or the
// row is masked off): a register move, no LDS round trip
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}

// Maximum over the 64 lanes of a wave (all active), in every lane: the same DPP
// pattern as the scan below with max in place of the sum (the lanes a pattern
// names none for take the identity), then lane 63's value.
__device__ __forceinline__ int wave_max(int x) {
    auto mv = [](int v, auto CTRL, auto ROWS) {
        return __builtin_amdgcn_update_dpp(INT_MIN, v, decltype(CTRL)::value, decltype(ROWS)::value, 0xF, false);
    };
    using R = std::integral_constant<int, 0xF>;
    x = max(x, mv(x, std::integral_constant<int, 0x111>{}, R{}));
    x = max(x, mv(x, std::integral_constant<int, 0x112>{}, R{}));
    x = max(x, mv(x, std::integral_constant<int, 0x114>{}, R{}));
    x = max(x, mv(x, std::integral_constant<int, 0x118>{}, R{}));
    x = max(x, mv(x, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{}));
    x = max(x, mv(x, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{}));
    return __builtin_amdgcn_readlane(x, 63);
}
__device__ __forceinline__ float wave_max(float x) {
    auto mv = [](float v, auto CTRL, auto ROWS) {
        return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v),
                                                          decltype(CTRL)::value, decltype(ROWS)::value, 0xF, false));
    };
    using R = std::integral_constant<int, 0xF>;
    x = fmaxf(x, mv(x, std::integral_constant<int, 0x111>{}, R{}));
    x = fmaxf(x, mv(x, std::integral_constant<int, 0x112>{}, R{}));
    x = fmaxf(x, mv(x, std::integral_constant<int, 0x114>{}, R{}));
    x = fmaxf(x, mv(x, std::integral_constant<int, 0x118>{}, R{}));
    x = fmaxf(x, mv(x, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{}));
    x = fmaxf(x, mv(x, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{}));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Inclusive sum over the 64 lanes of a wave (all active), in a fixed tree order
// (the same values give the same result in every call): prefix sums within each
// row of 16 lanes by shifts of 1, 2, 4 and 8, then the total of row 0 added to
// row 1 and of row 2 to row 3 (broadcast of lanes 15 and 47), then that of rows
// 0-1 to rows 2 and 3 (broadcast of lane 31).
__device__ __forceinline__ float wave_incl_scan(float x, int) {
    x += dpp_move<0x111, 0xF>(x);  // row_shr:1
    x += dpp_move<0x112, 0xF>(x);  // row_shr:2
    x += dpp_move<0x114, 0xF>(x);  // row_shr:4
    x += dpp_move<0x118, 0xF>(x);  // row_shr:8
    x += dpp_move<0x142, 0xA>(x);  // row_bcast:15, rows 1 and 3
    x += dpp_move<0x143, 0xC>(x);  // row_bcast:31, rows 2 and 3
    return x;
}

// Weights e_v = 2^(x_v c - m c) of one 8-element chunk (logits f, first index
// v0) summed in index order; lastpos becomes the chunk's last index of nonzero
// weight and elast its weight.
__device__ __forceinline__ float chunk_sum(const float (&f)[8], int v0, float c, float mc, float (&e)[8],
                                           int& lastpos, float& elast) {
    float cs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[j], c, -mc));
        cs += e[j];
        if (e[j] > 0.f) {
            lastpos = max(lastpos, v0 + j);
            elast = e[j];
        }
    }
    return cs;
}

// Elements [lo, hi) of a row one at a time from base: the first index where the
// running sum passes r (e_hit its weight), else -1; lastpos and the sum as above.
template <bool BF16>
__device__ __forceinline__ int walk_elems(const char* rp, int lo, int hi, float c, float mc, float base, float r,
                                          float& sum, int& lastpos, float& e_hit) {
    float x = base;
    for (int v = lo; v < hi; ++v) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(elem<BF16>(rp, v), c, -mc));
        x += e;
        if (e > 0.f) lastpos = max(lastpos, v);
        if (x > r) { e_hit = e; sum = x; return v; }
    }
    sum = x;
    return -1;
}

// Inverse transform draw for every masked row (one workgroup of 256 threads
// per row), after vocab_reduce has written the split triples. The split that
// holds the crossing is cut into its head (elements before the first aligned
// chunk, split 0 only), iterations of 64 consecutive chunks (wave i takes
// iterations i, i + 4, ..., one chunk per lane, so every load is coalesced)
// and its tail (last split only). The region totals go to LDS; one wave scans
// them in order and finds the region where the running sum passes the target.
// Inside an iteration, the first lane whose scan value passes walks its chunk
// element by element. When the split takes one round of loads (at most 4 NQ
// iterations), each wave keeps its chunks in registers, so the iteration is
// not read again.
template <bool BF16>
__global__ __launch_bounds__(256) void sample_locate(UArgs a) {
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const long long rows = (long long)a.B * a.S;
    const float c = a.c;
    __shared__ float sh_m, sh_z, sh_r, sh_u, sh_base;
    __shared__ int sh_k, sh_am, sh_region;
    __shared__ int wlast[4];
    __shared__ Triple tri[64];                   // n_vsplit <= 64
    __shared__ float tot[kSampleMaxIter + 2];    // head, iterations, tail
    // the mask, the split triples and the uniform in one round trip (an unmasked
    // row's triples are stale and never used)
    const uint8_t mk = a.mask_in[row];
    u32x4 tr = {0u, 0u, 0u, 0u};  // a Triple, as a register vector
    if (tid < a.n_vsplit) tr = *reinterpret_cast<const u32x4*>(a.part + (long long)tid * rows + row);
    float uu = 0.f;
    if (tid == 128) uu = a.uniforms[row];
    if (!mk) return;
    if (tid < a.n_vsplit) *reinterpret_cast<u32x4*>(&tri[tid]) = tr;
    if (tid == 128) sh_u = uu;
    __syncthreads();
    if (w == 0) {
        // wave 0, one split per lane (n_vsplit <= 64): the row max, its first
        // index (held by the first split whose max it is), the split weights
        // 2^((m_k - m) c) z_k and their in-order scan, whose total is Z; the
        // split where the scan passes u Z holds the draw
        const bool in = lane < a.n_vsplit;
        const float mk = in ? tri[lane].m : -INFINITY;
        const float m = wave_max(mk);
        const unsigned long long hm = __ballot(in && mk == m);
        const int am = hm ? __shfl(in ? tri[lane].a : INT_MAX, __builtin_ctzll(hm)) : INT_MAX;
        const float wk = m != -INFINITY && mk != -INFINITY ? tri[lane].z * __builtin_amdgcn_exp2f((mk - m) * c) : 0.f;
        const float inc = wave_incl_scan(wk, lane);
        float exc = __shfl_up(inc, 1);
        if (lane == 0) exc = 0.f;
        const float z = __shfl(inc, 63);
        float u = sh_u;
        u = u > 0.f ? fminf(u, 1.f) : 0.f;  // NaN and negatives count as 0
        const float t = u * z;
        int kk = -1;
        float r = INFINITY;
        if (m != -INFINITY) {
            const unsigned long long hit = __ballot(in && inc > t);
            if (hit) {
                kk = __builtin_ctzll(hit);
                r = t - __shfl(exc, kk);
            } else {  // not passed (u = 1, or rounding): the last split of nonzero weight
                const unsigned long long hp = __ballot(wk > 0.f);
                kk = hp ? 63 - __builtin_clzll(hp) : -1;
            }
        }
        if (lane == 0) {
            sh_m = m; sh_z = z; sh_r = r; sh_k = kk; sh_am = am;
        }
    }
    __syncthreads();
    const int k = sh_k;
    if (k < 0) {  // no logit of nonzero weight: the greedy result stands
        if (tid == 0) a.drawn[row] = Drawn{sh_am, 1.f / sh_z};
        return;
    }
    const float m = sh_m, z = sh_z, r = sh_r, mc = m * c;
    // the split's extent, cut exactly as in vocab_reduce
    constexpr int ES = BF16 ? 2 : 4;
    const char* rp = static_cast<const char*>(a.logits) + (long long)row * a.stride * ES;
    int a0 = (int)(((16u - (unsigned)(reinterpret_cast<uintptr_t>(rp) & 15u)) & 15u) / ES);
    if (a0 > a.V) a0 = a.V;
    const int nfull = (a.V - a0) / 8;
    const int per = (nfull + a.n_vsplit - 1) / a.n_vsplit;
    const int c0 = min(nfull, k * per), c1 = min(nfull, c0 + per);
    const int head = k == 0 ? a0 : 0;
    const int tail0 = a0 + nfull * 8;
    const int tail1 = k == a.n_vsplit - 1 ? a.V : tail0;
    const int NI = (c1 - c0 + 63) / 64;  // <= kSampleMaxIter (checked on the host)
    const char* body = rp + a0 * ES;
    int lastpos = -1;
    float scratch_sum, e_dummy;
    if (tid == 0) {
        walk_elems<BF16>(rp, 0, head, c, mc, 0.f, INFINITY, scratch_sum, lastpos, e_dummy);
        tot[0] = scratch_sum;
    }
    if (tid == 64) {
        walk_elems<BF16>(rp, tail0, tail1, c, mc, 0.f, INFINITY, scratch_sum, lastpos, e_dummy);
        tot[NI + 1] = scratch_sum;
    }
    // pass 1: region totals, NQ iterations of loads in flight per wave (lanes past
    // the split's end load its last chunk again and count nothing, so every load
    // is unconditional and they issue together). One round covers 4 NQ
    // iterations, 16384 logits: every split a drawing step plans, up to V = 2^20.
    constexpr int NQ = 8;
    u32x4 keep0[NQ], keep1[NQ];  // this wave's chunks of the last round of loads
    for (int G0 = w; G0 < NI; G0 += 4 * NQ) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            load_raw<BF16>(body, min(c0 + 64 * (G0 + 4 * q) + lane, c1 - 1), keep0[q], keep1[q]);
        float cs[NQ], incl[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int G = G0 + 4 * q;
            const int ch = c0 + 64 * G + lane;
            cs[q] = 0.f;
            if (G < NI && ch < c1) {
                float f[8];
                widen<BF16>(keep0[q], keep1[q], f);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(f[j], c, -mc));
                    cs[q] += e;
                    if (e > 0.f) lastpos = max(lastpos, a0 + ch * 8 + j);
                }
            }
        }
        // independent scans, so their shuffles overlap
#pragma unroll
        for (int q = 0; q < NQ; ++q) incl[q] = wave_incl_scan(cs[q], lane);
        if (lane == 63) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                if (G0 + 4 * q < NI) tot[1 + G0 + 4 * q] = incl[q];
        }
    }
    const int lp = wave_max(lastpos);
    if (lane == 0) wlast[w] = lp;
    __syncthreads();
    // the first region whose total takes the running sum past r: wave 0 scans the
    // totals 64 at a time; region i starts from base_i = carry + (exclusive scan)
    if (w == 0) {
        float carry = 0.f, base_hit = 0.f;
        int region = -1;
        for (int i0 = 0; i0 < NI + 2; i0 += 64) {
            const int i = i0 + lane;
            const float T = i < NI + 2 ? tot[i] : 0.f;
            const float inc = wave_incl_scan(T, lane);
            float exc = __shfl_up(inc, 1);
            if (lane == 0) exc = 0.f;
            const float bi = carry + exc;
            const unsigned long long hit = __ballot(i < NI + 2 && bi + T > r);
            if (hit) {
                const int l = __builtin_ctzll(hit);
                region = i0 + l;
                base_hit = __shfl(bi, l);
                break;
            }
            carry += __shfl(inc, 63);
        }
        if (lane == 0) {
            sh_region = region;
            sh_base = base_hit;
        }
    }
    __syncthreads();
    const int region = sh_region;
    const float base = sh_base;
    const int last_all = max(max(wlast[0], wlast[1]), max(wlast[2], wlast[3]));
    auto put = [&](int v, float e) {
        if (v >= 0) a.drawn[row] = Drawn{v, e / z};
        else a.drawn[row] = Drawn{sh_am, 1.f / z};
    };
    auto weight = [&](int v) { return __builtin_amdgcn_exp2f(__builtin_fmaf(elem<BF16>(rp, v), c, -mc)); };
    if (region < 0 || region == 0 || region == NI + 1) {
        if (tid == 0) {
            int v = -1, lpos = -1;
            float e = 0.f, sum;
            if (region == 0) v = walk_elems<BF16>(rp, 0, head, c, mc, base, r, sum, lpos, e);
            else if (region > 0) v = walk_elems<BF16>(rp, tail0, tail1, c, mc, base, r, sum, lpos, e);
            if (v < 0) {  // not passed (u = 1, or rounding): the last element of nonzero weight
                v = region < 0 ? last_all : lpos;
                if (v < 0) v = last_all;
                e = v >= 0 ? weight(v) : 0.f;
            }
            put(v, e);
        }
        return;
    }
    const int G = region - 1;
    if (w != (G & 3)) return;
    const int ch = c0 + 64 * G + lane;
    float e[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int lpos = -1;
    float elast = 0.f;  // the weight of lpos
    float cs = 0.f;
    if (ch < c1) {
        float f[8];
        if (NI <= 4 * NQ) {
            // iteration G = w + 4 q of the only round: its chunk is still in registers
            const int q = G >> 2;
            u32x4 r0 = keep0[0], r1 = keep1[0];
#pragma unroll
            for (int qq = 1; qq < NQ; ++qq)
                if (qq == q) {
                    r0 = keep0[qq];
                    r1 = keep1[qq];
                }
            widen<BF16>(r0, r1, f);
        } else {
            load_chunk<BF16>(body, ch, f);
        }
        cs = chunk_sum(f, a0 + ch * 8, c, mc, e, lpos, elast);
    }
    // the same sums as in pass 1, so lane 63 at least passes
    const float incl = wave_incl_scan(cs, lane);
    float excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.f;
    const unsigned long long hit = __ballot(base + incl > r);
    const int first = hit ? __builtin_ctzll(hit) : 63;
    int v = -1;
    float ev = 0.f;
    if (lane == first) {
        float x = base + excl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x += e[j];
            if (v < 0 && x > r && e[j] > 0.f) { v = a0 + ch * 8 + j; ev = e[j]; }
        }
        if (v < 0 && lpos >= 0) { v = lpos; ev = elast; }
    }
    if (__shfl(v, first) >= 0) {
        if (lane == first) put(v, ev);
        return;
    }
    // the passing lane's chunk has no weight (a scan rounding): the last weighted lane before it
    const unsigned long long below = __ballot(cs > 0.f && lane < first);
    if (below) {
        if (lane == 63 - __builtin_clzll(below)) put(lpos, elast);
    } else if (lane == 0) {
        put(last_all, last_all >= 0 ? weight(last_all) : 0.f);
    }
}

__global__ __launch_bounds__(64) void unmask_select(UArgs a) {
    const int b = blockIdx.x;
    const int l = threadIdx.x;
    const bool inb = l < a.S;
    const long long row = (long long)b * a.S + (inb ? l : 0);
    // The mask, the split triples and the draw are all requested before any of
    // them is used (one memory round trip, not one per dependent read). They are
    // read for every position of the sequence; an unmasked row's slots hold
    // stale values, which are never used.
    const uint8_t mk = a.mask_in[row];
    Drawn d{INT_MAX, 0.f};
    if (a.drawn) d = a.drawn[row];
    float m = -INFINITY, z = 0.f;
    int am = INT_MAX;
    const long long rows = (long long)a.B * a.S;
    for (int k0 = 0; k0 < a.n_vsplit; k0 += 8) {
        Triple t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (k0 + j < a.n_vsplit) t[j] = a.part[(long long)(k0 + j) * rows + row];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (k0 + j < a.n_vsplit) combine(m, am, z, t[j].m, t[j].a, t[j].z, a.c);
    }
    const bool masked = inb && mk != 0;
    float conf = masked ? 1.f / z : -INFINITY;
    if (masked && a.drawn) {
        am = d.a;
        conf = d.conf;
    }
    const unsigned long long mmask = __ballot(masked);
    const int M = __popcll(mmask);
    const int kmin = (M + a.steps_left - 1) / a.steps_left;
    const bool pass = masked && conf > a.gamma;
    const int npass = __popcll(__ballot(pass));
    bool commit;
    if (npass >= kmin) {
        commit = pass;
    } else {
        // rank among the masked positions: their confidences are read lane by
        // lane (a uniform index: a register read, not an LDS round trip each)
        int rank = 0;
        const int cbits = __float_as_int(conf);
        for (int j = 0; j < a.S; ++j) {
            if (!((mmask >> j) & 1ull)) continue;
            const float cj = __int_as_float(__builtin_amdgcn_readlane(cbits, j));
            rank += (cj > conf || (cj == conf && j < l)) ? 1 : 0;
        }
        commit = masked && rank < kmin;
    }
    const int ncommit = __popcll(__ballot(commit));
    if (inb) {
        const uint8_t old = a.mask_in[row];
        if (commit) a.tokens[row] = am;
        a.mask_out[row] = commit ? 0 : old;
        if (masked && a.conf) a.conf[row] = conf;
    }
    if (l == 0 && a.num_masked) a.num_masked[b] = M - ncommit;
}

// L_MD (section 2.2, Eq. (4)) from the (max, argmax, sum) triples of
// vocab_reduce at temperature 1: one workgroup of kNllThreads, thread t taking
// rows t, t + kNllThreads, ... The target, the mask and every split's triple of
// a row are requested before any is used, and a masked row's target logit as
// soon as the target and mask have arrived, so a row costs two memory round
// trips. Each thread sums its rows in row order, and the threads' sums are added
// in a fixed order (wave shuffles, then the waves in turn), in double: the loss
// does not depend on timing.
constexpr int kNllThreads = 1024;
template <bool BF16>
__global__ __launch_bounds__(kNllThreads) void nll_finish(UArgs a, const int* __restrict__ targets, float* nll,
                                                          float* loss, int* count) {
    const long long rows = (long long)a.B * a.S;
    double sum = 0.0;
    int n = 0;
    for (long long row = threadIdx.x; row < rows; row += kNllThreads) {
        const int y = targets[row];
        const uint8_t mk = a.mask_in[row];
        float m = -INFINITY, z = 0.f;
        int am = INT_MAX;
        float xt = 0.f;
        for (int k0 = 0; k0 < a.n_vsplit; k0 += 8) {
            Triple t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (k0 + j < a.n_vsplit) t[j] = a.part[(long long)(k0 + j) * rows + row];
            if (k0 == 0 && mk && y >= 0 && y < a.V)  // unmasked rows are not read
                xt = elem<BF16>(static_cast<const char*>(a.logits) + row * a.stride * (BF16 ? 2 : 4), y);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (k0 + j < a.n_vsplit) combine(m, am, z, t[j].m, t[j].a, t[j].z, a.c);
        }
        if (!mk) continue;
        const float v = y >= 0 && y < a.V ? m + __logf(z) - xt : __builtin_nanf("");
        if (nll) nll[row] = v;
        sum += (double)v;
        ++n;
    }
    // each wave halves its sums six times, then wave 0 adds the 16 wave sums in order
    for (int off = 32; off > 0; off >>= 1) {
        sum += __shfl_down(sum, off);
        n += __shfl_down(n, off);
    }
    constexpr int kWavesNll = kNllThreads / 64;
    __shared__ double ss[kWavesNll];
    __shared__ int sn[kWavesNll];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        ss[w] = sum;
        sn[w] = n;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        int c = 0;
        for (int k = 0; k < kWavesNll; ++k) {
            t += ss[k];
            c += sn[k];
        }
        *loss = c > 0 ? (float)(t / c) : 0.f;
        if (count) *count = c;
    }
}

}  // namespace

// Iterations of 64 chunks in the largest vocabulary split (an upper bound over
// the row alignments), which sample_locate's LDS table must hold.
static long long sample_iterations(const tt_conf_unmask_params& p, const UnmaskPlan& pl) {
    const long long nfull = (long long)p.V / 8;
    const long long per = (nfull + pl.n_vsplit - 1) / pl.n_vsplit;
    return (per + 63) / 64;
}

bool unmask_sample_fits(const tt_conf_unmask_params& p, const UnmaskPlan& pl) {
    return sample_iterations(p, pl) <= kSampleMaxIter;
}

UnmaskPlan plan_unmask(const tt_conf_unmask_params& p, int n_cu) {
    UnmaskPlan pl{};
    const long long rows = (long long)p.B * p.S;
    const int cu = n_cu > 0 ? n_cu : 256;
    // enough workgroups to cover the chip about 8 times, at least 2048 logits each
    long long want = rows > 0 ? (8LL * cu + rows - 1) / rows : 1;
    // a stochastic draw re-reads one split of each row: at most 16384 logits per
    // split (smaller splits measured slower: more reduction workgroups)
    if (p.uniforms && want < (p.V + 16383) / 16384) want = (p.V + 16383) / 16384;
    long long cap = (p.V + 2047) / 2048;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    if (want > 64) want = 64;
    pl.n_vsplit = (int)want;
    pl.ws_part = (size_t)pl.n_vsplit * (size_t)rows * sizeof(Triple);
    pl.ws_total = pl.ws_part + (p.uniforms ? (size_t)rows * sizeof(Drawn) : 0);
    return pl;
}

tt_status launch_unmask(const tt_conf_unmask_params& p, const UnmaskPlan& pl, void* ws, hipStream_t s) {
    UArgs a{};
    a.logits = p.logits;
    a.stride = p.logits_stride_row;
    a.mask_in = p.mask_in;
    a.mask_out = p.mask_out;
    a.tokens = p.tokens;
    a.conf = p.conf;
    a.num_masked = p.num_masked;
    a.part = static_cast<Triple*>(ws);
    a.B = p.B; a.S = p.S; a.V = p.V;
    a.n_vsplit = pl.n_vsplit;
    a.steps_left = p.steps_left;
    a.gamma = p.gamma;
    a.c = 1.44269504088896340736f / p.temperature;
    if (p.uniforms && !unmask_sample_fits(p, pl)) return TT_ERR_SHAPE;  // also refused in validation
    a.uniforms = p.uniforms;
    a.drawn = p.uniforms ? reinterpret_cast<Drawn*>(static_cast<char*>(ws) + pl.ws_part) : nullptr;
    const dim3 grid(p.B * p.S, pl.n_vsplit);
    if (p.dtype == TT_BF16)
        hipLaunchKernelGGL(vocab_reduce<true>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(vocab_reduce<false>, grid, dim3(256), 0, s, a);
    if (p.uniforms) {
        if (p.dtype == TT_BF16)
            hipLaunchKernelGGL(sample_locate<true>, dim3(p.B * p.S), dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(sample_locate<false>, dim3(p.B * p.S), dim3(256), 0, s, a);
    }
    hipLaunchKernelGGL(unmask_select, dim3(p.B), dim3(64), 0, s, a);
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

UnmaskPlan plan_nll(const tt_masked_nll_params& p, int n_cu) {
    tt_conf_unmask_params u{};
    u.B = p.B;
    u.S = p.S;
    u.V = p.V;
    return plan_unmask(u, n_cu);
}

tt_status launch_nll(const tt_masked_nll_params& p, const UnmaskPlan& pl, void* ws, hipStream_t s) {
    UArgs a{};
    a.logits = p.logits;
    a.stride = p.logits_stride_row;
    a.mask_in = p.mask;
    a.part = static_cast<Triple*>(ws);
    a.B = p.B; a.S = p.S; a.V = p.V;
    a.n_vsplit = pl.n_vsplit;
    a.c = 1.44269504088896340736f;  // temperature 1
    const dim3 grid(p.B * p.S, pl.n_vsplit);
    if (p.dtype == TT_BF16) {
        hipLaunchKernelGGL(vocab_reduce<true>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(nll_finish<true>, dim3(1), dim3(kNllThreads), 0, s, a, p.targets, p.nll, p.loss, p.count);
    } else {
        hipLaunchKernelGGL(vocab_reduce<false>, grid, dim3(256), 0, s, a);
        hipLaunchKernelGGL(nll_finish<false>, dim3(1), dim3(kNllThreads), 0, s, a, p.targets, p.nll, p.loss, p.count);
    }
    return hipGetLastError() == hipSuccess ? TT_OK : TT_ERR_HIP;
}

}  // namespace tt
