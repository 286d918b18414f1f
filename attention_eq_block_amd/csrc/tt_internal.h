// Internal declarations shared by the host layer and the kernel files of
// libtwotower_attn. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "twotower_attn.h"

namespace tt {

// ---- work decomposition of the bf16 attention path -------------------------
// One "pair" is (sequence b, kv head g, row block rb): the S*G query rows that
// share kv head g, cut into blocks of kRows rows. The key stream of a pair is
// its prefix in tiles of kTile keys followed by one tile of the S block keys.
// All pairs' tiles, laid end to end, are cut into n_seg segments of equal
// cost, one per workgroup (stream-K): a pair costs its tiles plus kPieceCost
// for starting a piece. A pair cut by a segment boundary is finished by a
// log-sum-exp merge of the per-segment partials.
constexpr int kTile = 64;   // keys per tile
constexpr int kRows = 256;  // query rows per workgroup (8 waves x 32 rows)
#ifndef TT_PIECE_COST
#define TT_PIECE_COST 3
#endif
constexpr int kPieceCost = TT_PIECE_COST;  // in tiles, measured on long prefixes

struct AttnPlan {
    int n_rb;      // row blocks per (b, g)
    int n_pairs;   // B * Hkv * n_rb
    int n_seg;     // workgroups of the main kernel (multiple of 8)
    int n_slots;   // partial slots: n_seg + n_pairs
    size_t ws_part_o;    // bytes of partial O
    size_t ws_part_lse;  // bytes of partial LSE
    size_t ws_units;     // bytes of the per-sequence unit offsets the merge reads
    size_t ws_total;
    int fin_split;       // thread groups the merge kernel splits a pair's partials over (1, 4 or 8)
};

AttnPlan plan_attn_bf16(const tt_block_attn_params& p, int n_cu);

// The allocation-free entry point's scratch: a device array of this many bytes
// inside the library; noalloc_scratch() returns its address on the current
// device (looked up on the first call there), or null with *st set.
constexpr size_t kNoallocScratchBytes = TT_NOALLOC_SCRATCH_BYTES;
void* noalloc_scratch(tt_status* st);
tt_status launch_attn_bf16(const tt_block_attn_params& p, const AttnPlan& plan, void* ws,
                           hipStream_t s);

tt_status launch_attn_f32(const tt_block_attn_params& p, hipStream_t s);

tt_status launch_kv_append(const tt_kv_append_params& p, hipStream_t s);

tt_status launch_lse_merge(int P, const float* O_parts, const float* lse_parts, int B, int S, int Hq,
                           int d, void* O_out, int o_dtype, float* lse_out, hipStream_t s);

// sample_locate keeps one total per 64 chunks of a vocabulary split in LDS: with
// at most 64 splits this bounds a sampled vocabulary at 64 * 4096 * 512 = 2^27.
constexpr int kSampleMaxIter = 4096;

struct UnmaskPlan {
    int n_vsplit;
    size_t ws_part;  // split triples; the drawn tokens follow when sampling
    size_t ws_total;
};
UnmaskPlan plan_unmask(const tt_conf_unmask_params& p, int n_cu);
// with uniforms: the largest vocabulary split fits sample_locate's table
bool unmask_sample_fits(const tt_conf_unmask_params& p, const UnmaskPlan& plan);
UnmaskPlan plan_nll(const tt_masked_nll_params& p, int n_cu);
tt_status launch_unmask(const tt_conf_unmask_params& p, const UnmaskPlan& plan, void* ws,
                        hipStream_t s);
tt_status launch_nll(const tt_masked_nll_params& p, const UnmaskPlan& plan, void* ws, hipStream_t s);

// prefix length of sequence b as the kernels read it
__device__ __forceinline__ int clamp_len(int L, int Lmax) { return L < 0 ? 0 : (L > Lmax ? Lmax : L); }

}  // namespace tt
