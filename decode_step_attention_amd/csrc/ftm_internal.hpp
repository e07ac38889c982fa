// ftm_internal.hpp -- what the host dispatcher and the gfx950 kernels share:
// the launch parameters and the launcher entry points.  Not part of the
// public C ABI (include/ftm.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ftm {

enum KvKind : int { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2, KV_I8 = 3 };

// Everything one decode step needs, by value into the kernels.
struct Params {
    const void* q;          // [B, H, D] act
    const void* k_new;      // [B, Hkv, D] act
    const void* v_new;      // [B, Hkv, D] act
    const void* bias;       // [(H + 2 Hkv) D] act or null
    void* k_cache;          // [B, Hkv, Lmax, D] kv; paged: [n_pages, Hkv, P, D]
    void* v_cache;          // same layout as k_cache
    const int32_t* seq_lens;// [B] or null
    float* kv_scales;       // [2, B, Hkv, Lmax] (INT8) or null; paged: [2, n_pages, Hkv, P]
    void* out;              // [B, H, D] act
    float* ws_o;            // [B, H, S, D]  un-normalised partial outputs
    float* ws_ml;           // [B, H, S, 2]  partial (max, sum), log2 domain
    int B, Lmax, step, H, Hkv, G;
    int n_hg;               // query-head groups per KV head (ceil(G / group tile))
    int chunk;              // positions per split chunk (multiple of the tile)
    int S;                  // chunks per sequence at length `step`
    int direct;             // 1: single pass writes `out`; 0: write partials
    float qscale;           // log2(e) / sqrt(D), folded into the query
    // balanced grouped-query schedule (grid of S workgroups)
    int balanced;           // 1: grouped-query pass on the matrix cores
    int* counters;          // [units] finished-piece counts, zero between calls
    int range_min;          // fewest 16-row tiles a workgroup's range holds
    int unit_cost;          // virtual tiles charged per unit (segment prologue and epilogue)
    int skew_a, skew_b;     // tiles per round for each older / younger wave of a workgroup
    // paged cache (block_table null: contiguous [B, Hkv, Lmax, D] cache)
    const int32_t* block_table;   // [B, max_pages]: page of positions [i P, (i+1) P)
    int page_shift;         // log2(P), P >= 16
    int max_pages;          // block-table row length
    int n_pages;            // pages in the pool
};

// Tuning variables, read from the environment once (ftm_tuning_reload reads
// them again).  0 or -1 means "not set": the built-in choice applies.
struct Tuning {
    int validate;           // FTM_VALIDATE=1: blocking host check of seq_lens
    int waves;              // FTM_WAVES: 4 or 16 waves per single-head workgroup
    int split_chunk;        // FTM_SPLIT_CHUNK: positions per split chunk
    int gqa_valu;           // FTM_GQA_VALU=1: grouped heads on the vector pass
    int gqa_blocks_per_cu;  // FTM_GQA_BLOCKS_PER_CU: 1..16
    int gqa_unit_cost;      // FTM_GQA_UNIT_COST: 0..64, -1 unset
    int gqa_skew_a, gqa_skew_b;  // FTM_GQA_SKEW=a,b: 1..16 each
    int qkv_column_tiles;   // FTM_QKV_COLUMN_TILES: 1..4
    int qkv_k_split;        // FTM_QKV_K_SPLIT: 1 (one pass) or 2..4, -1 unset
};
const Tuning& tuning();

// Group tile (query heads served by one pass over a KV head) for G heads.
int group_tile(int G);
// Positions one workgroup of `nw` waves of the vector-ALU pass covers per
// streaming iteration.
int tile_rows(int kv, int head_dim, int group_tile, int nw);
// Whether a pass of `group_tile` heads over this cache type runs on the
// matrix cores with the balanced schedule (fp16/bf16 caches, 4 or 8 heads,
// batch <= 256; FTM_GQA_VALU=1 turns it off).
bool use_gqa_mfma(int kv, int group_tile, int batch);
// Workgroups per CU of the grouped-query pass.
int gqa_blocks_per_cu();
// Virtual tiles the range schedule charges per unit.
int gqa_unit_cost();
// Tiles per round for an older and a younger wave of the grouped-query pass.
void gqa_skew(int& a, int& b);
// Most pieces one unit is cut into by the range schedule (the merge of a
// unit's pieces reads them four per round).
constexpr int kGqaMaxPieces = 128;
// Whether the 16-wave workgroup is built for this cache type and group tile.
bool wide_ok(int kv, int group_tile);

// The fused QKV projection: y = x W^T (+ bias), split into q, k_new, v_new.
struct QkvParams {
    const void* x;          // [B, hidden] act
    const void* w;          // [(H + 2 Hkv) D, hidden] act
    const void* bias;       // [(H + 2 Hkv) D] act or null
    void* q;                // [B, H, D] act
    void* k_new;            // [B, Hkv, D] act
    void* v_new;            // [B, Hkv, D] act
    int B, hidden, H, Hkv, D;
    float* ws;              // k-split partial sums (qkv_split_workspace bytes) or null
    int* counters;          // k-split: one count per 128-feature column, zero between calls
};

// Prefill: the whole prompt of every sequence.
struct PrefillParams {
    const void* q;          // [B, S, H, D] act
    const void* k_new;      // [B, S, Hkv, D] act
    const void* v_new;      // [B, S, Hkv, D] act
    const void* bias;       // [(H + 2 Hkv) D] act or null
    void* k_cache;          // [B, Hkv, Lmax, D] kv (= act)
    void* v_cache;
    const int32_t* seq_lens;// [B] prompt lengths or null (all S)
    void* out;              // [B, S, H, D] act
    int B, S, Lmax, H, Hkv;
    float qscale;           // log2(e) / sqrt(D)
    // paged cache (block_table non-null): k_cache/v_cache are pools
    // [n_pages, Hkv, 2^page_shift, D], position t of sequence b is row
    // t mod P of page block_table[b * max_pages + t / P]
    const int32_t* block_table;
    int page_shift, max_pages, n_pages;
    // INT8 cache: its scales ([2, B, Hkv, Lmax], or [2, n_pages, Hkv, P]
    // paged), and the staging the attention reads: the prompt's codes as
    // fp16 [B, Hkv, S, D] and their scales [B, Hkv, S], K and V
    float* kv_scales;
    void* stage_k;
    void* stage_v;
    float* stage_ks;
    float* stage_vs;
    // float caches with a bias: b_q . k of every prompt row and query head,
    // [B, H, S] fp32, written by the append and read by the attention
    float* bterm;
};

hipError_t launch_attention(const Params& p, int kv, int head_dim, int gtile, int nw, hipStream_t s);
// kv: KV_F16 or KV_BF16; head_dim 64 or 128.  Two launches: append, then attention.
// The prompt's K/V rows into the cache, then the causal attention over them.
hipError_t launch_prefill_append(const PrefillParams& p, int kv, int head_dim, hipStream_t s);
hipError_t launch_prefill_attention(const PrefillParams& p, int kv, int head_dim, hipStream_t s);
// INT8: the append quantises the prompt's rows into the cache and the
// staging; the attention then runs on the staging (p.stage_*).
hipError_t launch_prefill_append_i8(const PrefillParams& p, int head_dim, hipStream_t s);
hipError_t launch_prefill_attention_i8(const PrefillParams& p, int head_dim, hipStream_t s);
// act: KV_F16 or KV_BF16; B <= 64, hidden a multiple of 256, (H + 2 Hkv) D a multiple of 16.
hipError_t launch_qkv_proj(const QkvParams& p, int act, int n_cu, hipStream_t s);
// Workspace bytes and counters the projection of this shape uses (0 and 0
// when it runs in one pass).
size_t qkv_split_workspace(const QkvParams& p, int n_cu, size_t* n_counters);
hipError_t launch_combine(const Params& p, int kv, int head_dim, hipStream_t s);
// Sets n ints at `dst` to zero with a kernel on `s` (no memset node, so it
// may also be recorded into a graph).
hipError_t launch_zero_ints(int* dst, size_t n, hipStream_t s);

// Scratch of the allocation-free decode call: a fixed device array of
// kStaticScratchBytes per GPU, the grouped-query counters in its first
// kStaticCounterInts ints and the split partials after them.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
constexpr size_t kStaticCounterInts = 16384;
constexpr size_t kStaticPartialBytes = kStaticScratchBytes - kStaticCounterInts * sizeof(int);
// The device address of the current device's scratch (taken once per
// device; the first call also clears the counters with a kernel on `s`).
hipError_t static_scratch(int device, hipStream_t s, void** ptr);

}  // namespace ftm
