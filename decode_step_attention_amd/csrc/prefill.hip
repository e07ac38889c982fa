// prefill.hip -- gfx950 kernels for prefill: the whole prompt of every
// sequence in one step.  The prompt is processed in parallel where decode
// goes token by token ([lpnh.cn/news/2765398] section 1.1): its K/V rows
// are appended to the cache, and every position t attends causally to
// positions [0, t] of its KV head.
//
// prefill_append_kernel: the prompt's K/V rows, with the bias added in fp32,
//   rounded to nearest even into the cache (one 16-byte slice per thread),
//   and, with a bias, the terms b_q . k of every row and query head.
// prefill_attn_kernel: one workgroup of 4 waves owns 128 query positions of
//   one query head; each wave owns two blocks of 16.  Keys [0, last query]
//   go through LDS in 64-key tiles, loaded straight from the cache into LDS
//   (16 bytes per lane) and swizzled against bank conflicts.  Each wave
//   takes 32 keys per step: S^T = K Q^T on the matrix cores
//   (v_mfma_f32_16x16x32), which leaves each lane with four keys of one
//   query, already the B-operand layout of P^T; the online softmax in the
//   query's own lanes; and O^T += V^T P^T, with V read down its columns by the
//   transposing LDS read.  The steps are software-pipelined: the next
//   step's S^T is computed between this step's exponentials.  The query
//   enters exactly as stored (kept in registers) and the bias term b_q . k,
//   the same for every query of a head, once per key, so every product is
//   exact in fp32; log2(e)/sqrt(D) scales the fp32 scores.  fp16 weights
//   are rounded once to nearest (11 significant bits, a relative error of
//   at most 2^-12 each); bf16 weights, and those over INT8 codes, enter as
//   hi/lo halves, so about 16 (bf16) or 22 (fp16) bits of each reach the
//   accumulators, as in the decode pass.  Workgroups with the most keys are
//   launched first.
#include <cstdlib>

#include "gfx950.hpp"

namespace ftm {
namespace {

constexpr int kQB = 2;                    // 16-query blocks per wave
constexpr int kPQ = 4 * 16 * kQB;         // query positions per workgroup
constexpr int kPK = 64;                   // key positions per LDS tile
constexpr float kNegInfP = -__builtin_inff();
constexpr float kLazy = 8.0f;             // log2 headroom of the softmax reference
// The INT8 staging holds V codes times this power of two and V scales
// divided by it (see prefill_append_i8_kernel).
constexpr float kVStageGain = 8.0f;

// Grid (ceil(S / RPB) Hkv, B): a block owns RPB consecutive positions of
// one (sequence, KV head), so its cache rows, and its bias terms per query
// head, are each one contiguous run; a thread owns 8 elements (16 bytes) of
// one row, the SL threads of a row are adjacent lanes.
template <int KV, int D, bool PG>
__global__ void __launch_bounds__(256) prefill_append_kernel(const PrefillParams p) {
    constexpr int SL = D / 8;               // threads per head row
    constexpr int RPB = 256 / SL;           // rows per block
    const int b = blockIdx.y;
    const int nt = (p.S + RPB - 1) / RPB;
    const int j = (int)blockIdx.x / nt;
    const int t = ((int)blockIdx.x - j * nt) * RPB + (int)threadIdx.x / SL;
    const int e0 = ((int)threadIdx.x % SL) * 8;
    const int Sb = p.seq_lens ? p.seq_lens[b] : p.S;
    if (Sb < 1 || Sb > p.S || t >= Sb) return;         // invalid length: no append (whole rows return)
    const size_t src = (((size_t)b * p.S + t) * p.Hkv + j) * D + e0;
    size_t dst;
    if constexpr (PG) {
        // row t mod P of the page the table names; no append into a page
        // outside the pool
        const int pg = p.block_table[(size_t)b * p.max_pages + (t >> p.page_shift)];
        if (pg < 0 || pg >= p.n_pages) return;
        dst = ((((size_t)pg * p.Hkv + j) << p.page_shift) + (t & ((1 << p.page_shift) - 1))) * D + e0;
    } else {
        dst = (((size_t)b * p.Hkv + j) * p.Lmax + t) * D + e0;
    }
    const u32x4 kraw = *(const u32x4*)((const uint16_t*)p.k_new + src);
    const u32x4 vraw = *(const u32x4*)((const uint16_t*)p.v_new + src);
    u32x4 kb = u32x4{0u, 0u, 0u, 0u}, vb = kb;
    if (p.bias) {
        kb = *(const u32x4*)((const uint16_t*)p.bias + (size_t)(p.H + j) * D + e0);
        vb = *(const u32x4*)((const uint16_t*)p.bias + (size_t)(p.H + p.Hkv + j) * D + e0);
    }
    float ks[8];                            // the stored K values, as fp32
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        float x[8], bx[8];
        Elem16<KV>::unpack(which ? vraw : kraw, x);
        Elem16<KV>::unpack(which ? vb : kb, bx);
        uint32_t hb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float y = x[e] + bx[e];   // one fp32 rounding (an absent bias adds +0)
            hb[e] = KV == KV_F16 ? float_to_half_bits(y) : float_to_bf16_bits(y);
            if (which == 0) ks[e] = KV == KV_F16 ? half_bits_to_float(hb[e]) : bf16_bits_to_float(hb[e]);
        }
        *(u32x4*)((uint16_t*)(which ? p.v_cache : p.k_cache) + dst) =
            u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
    }
    // the bias terms b_q . k of this row for the query heads of KV head j:
    // exact products of the stored K and the query bias, summed in fp32 over
    // this thread's 8 elements and then over the SL threads of the row
    // (adjacent lanes of one DPP row, SL a power of two)
    if (p.bterm) {
        const int G = p.H / p.Hkv;
        for (int gi = 0; gi < G; ++gi) {
            const int h = j * G + gi;
            float bq[8];
            Elem16<KV>::unpack(*(const u32x4*)((const uint16_t*)p.bias + (size_t)h * D + e0), bq);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = __builtin_fmaf(bq[e], ks[e], d);
            d = group_sum<SL>(d);           // the row's SL lanes, by DPP
            if (e0 == 0) p.bterm[((size_t)b * p.H + h) * p.S + t] = d;
        }
    }
}

// The decode step's INT8 codes of 16 elements of a row with scale s:
// rint(x / s) with the IEEE quotient, clamped to [-127, 127]; s = 0 gives
// zeros.  Fast path: with r = 1/s (one IEEE division) the product x r lies
// within 3 |x/s| 2^-24 <= 2.3e-5 of the rounded quotient (|x/s| <= 127), so
// where x r is more than 2^-14 away from every half-integer both round to
// the same integer.  A thread with any element closer than that (or a
// non-finite product) takes the IEEE quotients for all 16.
__device__ __forceinline__ void quantize16_i8(const float* x, float scale, float* cq) {
    if (scale != 0.0f) {
        const float r = 1.0f / scale;
        bool fast = true;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float q0 = x[e] * r;
            cq[e] = rintf(q0);
            fast = fast && fabsf(q0 - cq[e]) < 0.5f - 0x1p-14f;   // false for NaN
        }
        if (!fast) {
#pragma unroll
            for (int e = 0; e < 16; ++e) cq[e] = rintf(x[e] / scale);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) cq[e] = fminf(fmaxf(cq[e], -127.0f), 127.0f);
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) cq[e] = 0.0f;
    }
}

// INT8 cache: the prompt's rows, bias added in fp32 and quantised by the
// decode step's rule (s = absmax / 127 by IEEE division, code = rint(x / s)
// clamped to [-127, 127], a zero row keeps s = 0), into the cache and its
// scales, and into the staging the attention reads: the codes as fp16 (exact)
// and the scales, contiguous.  Grid (ceil(S / RPB) Hkv, B): a block owns RPB
// consecutive positions of one (sequence, KV head), so its code rows,
// staging rows and scales are each one contiguous run; a thread owns 16
// elements of one row, the SL threads of a row are adjacent lanes.  All of
// a thread's loads are issued before any store.
template <int D, bool PG>
__global__ void __launch_bounds__(256) prefill_append_i8_kernel(const PrefillParams p) {
    constexpr int SL = D / 16;              // threads per head row
    constexpr int RPB = 256 / SL;           // rows per block
    const int b = blockIdx.y;
    const int nt = (p.S + RPB - 1) / RPB;
    const int j = (int)blockIdx.x / nt;
    const int t = ((int)blockIdx.x - j * nt) * RPB + (int)threadIdx.x / SL;
    const int e0 = ((int)threadIdx.x % SL) * 16;
    const int Sb = p.seq_lens ? p.seq_lens[b] : p.S;
    if (Sb < 1 || Sb > p.S || t >= Sb) return;         // invalid length: no append
    const size_t src = (((size_t)b * p.S + t) * p.Hkv + j) * D + e0;
    u32x4 raw[2][2], braw[2][2];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* in = (const uint16_t*)(which ? p.v_new : p.k_new) + src;
        raw[which][0] = *(const u32x4*)in;
        raw[which][1] = *(const u32x4*)(in + 8);
        if (p.bias) {
            const uint16_t* bb = (const uint16_t*)p.bias + (size_t)(p.H + which * p.Hkv + j) * D + e0;
            braw[which][0] = *(const u32x4*)bb;
            braw[which][1] = *(const u32x4*)(bb + 8);
        }
    }
    // destination row in the cache (-1: a page outside the pool, no append)
    long long crow;                         // row index in rows of D codes
    size_t srow;                            // scale index within K's (or V's) half
    if constexpr (PG) {
        const int pg = p.block_table[(size_t)b * p.max_pages + (t >> p.page_shift)];
        const bool ok = pg >= 0 && pg < p.n_pages;
        const size_t r = (((size_t)(ok ? pg : 0) * p.Hkv + j) << p.page_shift) + (t & ((1 << p.page_shift) - 1));
        crow = ok ? (long long)r : -1;
        srow = r;
    } else {
        crow = (long long)(((size_t)b * p.Hkv + j) * p.Lmax + t);
        srow = (size_t)crow;
    }
    const size_t half = PG ? (size_t)p.n_pages * p.Hkv << p.page_shift : (size_t)p.B * p.Hkv * p.Lmax;
    const size_t stage_row = ((size_t)b * p.Hkv + j) * p.S + t;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        float x[16];
        Elem16<KV_F16>::unpack(raw[which][0], x);
        Elem16<KV_F16>::unpack(raw[which][1], x + 8);
        if (p.bias) {
            float bx[16];
            Elem16<KV_F16>::unpack(braw[which][0], bx);
            Elem16<KV_F16>::unpack(braw[which][1], bx + 8);
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = x[e] + bx[e];   // one fp32 rounding
        }
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
        for (int off = 1; off < SL; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        const float scale = amax / 127.0f;
        float cq[16];
        quantize16_i8(x, scale, cq);
        uint32_t w[4], hq[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {       // bytes 0 of four codes -> one word
            const uint32_t lo = __builtin_amdgcn_perm((uint32_t)(int32_t)cq[4 * k + 1], (uint32_t)(int32_t)cq[4 * k],
                                                      0x0c0c0400u);
            const uint32_t hi = __builtin_amdgcn_perm((uint32_t)(int32_t)cq[4 * k + 3], (uint32_t)(int32_t)cq[4 * k + 2],
                                                      0x0c0c0400u);
            w[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        const float gain = which ? kVStageGain : 1.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)         // integers of at most 11 bits: exact in fp16 under any rounding
            hq[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(cq[2 * k] * gain, cq[2 * k + 1] * gain));
        if (crow >= 0) {
            *(u32x4*)((int8_t*)(which ? p.v_cache : p.k_cache) + (size_t)crow * D + e0) = u32x4{w[0], w[1], w[2], w[3]};
            if (e0 == 0) p.kv_scales[which * half + srow] = scale;
        }
        uint16_t* st = (uint16_t*)(which ? p.stage_v : p.stage_k) + stage_row * D + e0;
        *(u32x4*)st = u32x4{hq[0], hq[1], hq[2], hq[3]};
        *(u32x4*)(st + 8) = u32x4{hq[4], hq[5], hq[6], hq[7]};
        // V is staged as code x kVStageGain with its scale / kVStageGain: the
        // attention puts each softmax weight (at most 2^kLazy) times its key's
        // staged V scale into fp16, and a row of fp16 values plus bias can
        // reach an absmax of 131008 (scale 1031.6); divided by 8 that product
        // stays below 33013 for every finite input.  Only a power of two
        // moves between the two factors of each product.
        if (e0 == 0) (which ? p.stage_vs : p.stage_ks)[stage_row] = which ? scale * (1.0f / kVStageGain) : scale;
    }
}

// Whether the softmax weights enter P.V as hi + lo halves.  bf16 keeps 8
// significant bits, too few for the output bar when one key dominates.
// fp16 keeps 11, enough with one rounding for values of the prompt's size;
// the INT8 staging (SC) multiplies each weight by its key's V scale and
// then by codes up to 127 (outputs of a few units, a sharp softmax), where
// one rounding measured 2.9e-3 against the 2e-3 bar, so it keeps the split.
template <int KV, bool SC> constexpr bool kWeightSplit = KV == KV_BF16 || SC;
// Whether the running sum of the weights is taken on the matrix cores, as
// P.1 (an all-ones A operand) accumulated beside O: when the weights enter
// P.V once rounded, the sum then uses the very weights the output does,
// and it costs one MFMA per query block and step instead of 16 adds.
template <int KV, bool SC> constexpr bool kSumOnMfma = !kWeightSplit<KV, SC>;

// The softmax weights (0 <= x <= 2^kLazy) as P operands.  Without a split
// (fp16): x rounded to nearest, lo unused.  With one: hi keeps the leading
// 11 (fp16) or 8 (bf16) significant bits by truncation, so it converts
// exactly (for x at least 2^-14 in fp16) and the fp32 residual x - hi is
// exact; lo is that residual rounded to the half type.
template <int KV, bool SPLIT>
__device__ __forceinline__ void split_weights(const float* x, typename Mfma<KV>::vec8& hi,
                                              typename Mfma<KV>::vec8& lo) {
    constexpr uint32_t kKeep = KV == KV_F16 ? 0xFFFFE000u : 0xFFFF0000u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if constexpr (KV == KV_F16 && !SPLIT) {
            hi[i] = (_Float16)x[i];
            lo[i] = (_Float16)0.0f;
        } else if constexpr (KV == KV_F16) {
            const float h = __uint_as_float(__float_as_uint(x[i]) & kKeep);
            hi[i] = (_Float16)h;
            lo[i] = (_Float16)(x[i] - h);
        } else {
            const float h = __uint_as_float(__float_as_uint(x[i]) & kKeep);
            hi[i] = (__bf16)h;
            lo[i] = (__bf16)(x[i] - h);
        }
    }
}

// SC: the K/V rows are INT8 codes staged as fp16 (p.k_cache / p.v_cache
// point at the staging, p.Lmax = S) with one scale per key: each raw score
// is multiplied by its key's K scale and each weight, for O only, by its
// key's V scale (the sum of the weights is taken unscaled).
template <int KV, int D, bool PG, bool BIAS, bool SC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
prefill_attn_kernel(const PrefillParams p) {
    using MF = Mfma<KV>;
    typedef typename MF::vec8 vec8;
    constexpr int ROW = D * 2;              // bytes per cache row
    constexpr int NCH = ROW / 16;           // 16-byte chunks per row
    constexpr int TILE = kPK * ROW;         // bytes per K (or V) tile
    constexpr int NI = TILE / 1024 / 4;     // tile loads per wave, each of K and V (1 KiB each)
    constexpr int KK = D / 32;              // S^T: MFMA steps over the head dim
    constexpr int DT = D / 16;              // O^T: 16-row tiles
    static_assert(NI >= 1 && TILE % 4096 == 0, "tile loads cover the tile");
    // Tiles are stored unpadded, filled by loads straight from memory into
    // LDS (lane i of a load writes bytes 16i..16i+15 of its 1 KiB), two
    // buffers deep.  Chunk c of row r sits in slot c ^ kswz(r) (K) or
    // c ^ vswz(r) (V), so the 16-byte reads of 16 rows (K) and the
    // transposing reads of 4 rows x 32 bytes per 16 lanes (V) hit distinct
    // banks.
    // (four separate arrays, each named at compile time wherever it is
    // used, so that the compiler can tell the buffer being filled from the
    // one being read and need not wait for the fill before the reads)
    __shared__ __attribute__((aligned(1024))) unsigned char ktile0[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char vtile0[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char ktile1[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char vtile1[TILE];
    // SC: each wave's own copy of a tile's 64 key scales (one 4-byte load
    // per lane), loaded with the K (or V) tile.  Float caches with a bias:
    // the K buffers hold the tile's 64 bias terms b_q . k instead.
    constexpr bool kBiasTerms = BIAS && !SC;
    constexpr int SCB = SC ? 4 * 64 * 4 : (kBiasTerms ? 4 * 64 * 4 : 16);
    __shared__ __attribute__((aligned(16))) unsigned char kscl0[SCB];
    __shared__ __attribute__((aligned(16))) unsigned char vscl0[SCB];
    __shared__ __attribute__((aligned(16))) unsigned char kscl1[SCB];
    __shared__ __attribute__((aligned(16))) unsigned char vscl1[SCB];
    auto kswz = [](int r) { return (r * NCH / 16) & (NCH - 1); };
    auto vswz = [](int r) { return 2 * ((r * NCH / 16) & (NCH / 2 - 1)); };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;                // MFMA layout: k group / key quad
    const int n = lane & 15;                // MFMA layout: key row (A) / query column (B, C)
    // blockIdx.x = r + B Hkv gi with r = b Hkv + j: the G query heads of one
    // KV head sit B Hkv apart, which keeps them on one L2 when B Hkv is a
    // multiple of the eight dispatch slots; blockIdx.y counts query blocks
    // from the last (the most keys) down, so the longest blocks go first
    const int G = p.H / p.Hkv;
    const int R = p.B * p.Hkv;
    const int r = blockIdx.x % R;
    const int b = r / p.Hkv;
    const int j = r - b * p.Hkv;
    const int h = j * G + blockIdx.x / R;
    const int qblk = gridDim.y - 1 - blockIdx.y;
    const int Sb = __builtin_amdgcn_readfirstlane(p.seq_lens ? p.seq_lens[b] : p.S);
    const int t0 = qblk * kPQ;
    if (Sb < 1 || Sb > p.S) {               // invalid length: NaN rows
        for (int idx = tid; idx < kPQ * D; idx += 256) {
            const int t = t0 + idx / D;
            if (t < p.S) {
                const size_t o = (((size_t)b * p.S + t) * p.H + h) * D + idx % D;
                ((uint16_t*)p.out)[o] = KV == KV_F16 ? 0x7e00u : 0x7fc0u;
            }
        }
        return;
    }
    if (t0 >= Sb) return;                   // past the prompt: nothing to do
    if (PG || (SC && p.block_table != nullptr)) {
        // a page outside the pool among the sequence's pages: NaN rows (the
        // staged INT8 path reads contiguous staging but keeps the table for
        // this check)
        const int npg = (Sb + (1 << p.page_shift) - 1) >> p.page_shift;
        bool bad = false;
        for (int i = lane; i < npg; i += 64) {
            const int pg = p.block_table[(size_t)b * p.max_pages + i];
            bad = bad || pg < 0 || pg >= p.n_pages;
        }
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
            for (int idx = tid; idx < kPQ * D; idx += 256) {
                const int t = t0 + idx / D;
                if (t < Sb) {
                    const size_t o = (((size_t)b * p.S + t) * p.H + h) * D + idx % D;
                    ((uint16_t*)p.out)[o] = KV == KV_F16 ? 0x7e00u : 0x7fc0u;
                }
            }
            return;
        }
    }
    const int kend = min(t0 + kPQ, Sb);     // keys [0, kend) are needed
    const int tq = t0 + wave * 16 * kQB;    // this wave's first query

    // K/V rows [0, kend) of (b, j) from the cache; rows past kend read as
    // zero (and the V rows past kend are cleared below as well)
    const size_t row0 = PG ? 0 : ((size_t)b * p.Hkv + j) * p.Lmax;
    const auto krs = make_rsrc((const char*)p.k_cache + row0 * ROW, (uint32_t)kend * ROW);
    const auto vrs = make_rsrc((const char*)p.v_cache + row0 * ROW, (uint32_t)kend * ROW);
    const size_t srow0 = ((size_t)b * p.Hkv + j) * p.Lmax;
    const auto ksr = make_rsrc(SC ? (const char*)(p.stage_ks + srow0)
                                  : kBiasTerms ? (const char*)(p.bterm + ((size_t)b * p.H + h) * p.S) : nullptr,
                               SC || kBiasTerms ? (uint32_t)kend * 4 : 0u);
    const auto vsr = make_rsrc(SC ? (const char*)(p.stage_vs + srow0) : nullptr, SC ? (uint32_t)kend * 4 : 0u);
    // one 64-key tile of K or V into LDS: NI loads per lane; load u of this
    // wave fills tile bytes base(u) .. +1023, lane i bytes base + 16 i .. +15,
    // which hold chunk slot ^ swz(row) of cache row k0 + row
    int koffs[NI], voffs[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
        const int base = (wave * NI + u) * 1024;
        const int row = (base + lane * 16) / ROW;
        const int slot = (base + lane * 16) % ROW / 16;
        koffs[u] = row * ROW + (slot ^ kswz(row)) * 16;
        voffs[u] = row * ROW + (slot ^ vswz(row)) * 16;
    }
    // Paged: the rows a wave loads per tile (NI loads of 1 KiB, 16
    // consecutive rows starting at a multiple of 16; page sizes are at least
    // 16) lie in one page, so the wave's loads share one descriptor over
    // that page's rows below kend, built from one table entry read through
    // the scalar cache.  A page past the table or outside the pool reads as
    // zeros (the sequence's rows are then NaN, see above).
    static_assert(NI * (1024 / ROW) == 16, "a wave loads 16 rows per tile");
    const __attribute__((address_space(4))) int32_t* tbl =
        (const __attribute__((address_space(4))) int32_t*)(PG ? p.block_table + (size_t)b * p.max_pages : nullptr);
    auto issue = [&](const bool is_v, int k0, unsigned char* dst, const int* offs, unsigned char* sdst) {
        if constexpr (SC)
            buffer_load_lds4(is_v ? vsr : ksr, sdst + wave * 256, lane * 4, __builtin_amdgcn_readfirstlane(k0 * 4));
        if constexpr (kBiasTerms) {
            if (!is_v) buffer_load_lds4(ksr, sdst + wave * 256, lane * 4, __builtin_amdgcn_readfirstlane(k0 * 4));
        }
        if constexpr (!PG) {
            const auto rs = is_v ? vrs : krs;
            const int so = __builtin_amdgcn_readfirstlane((int)((uint32_t)k0 * ROW));
#pragma unroll
            for (int u = 0; u < NI; ++u) buffer_load_lds16(rs, dst + (wave * NI + u) * 1024, offs[u], so);
        } else {
            const char* pool = (const char*)(is_v ? p.v_cache : p.k_cache);
            const int key0 = __builtin_amdgcn_readfirstlane(k0 + wave * 16);
            const int pi = key0 >> p.page_shift;
            const int pg = tbl[min(pi, p.max_pages - 1)];
            const bool ok = pi < p.max_pages && pg >= 0 && pg < p.n_pages;
            const int prow0 = pi << p.page_shift;
            const int nrows = ok ? max(0, min(kend - prow0, 1 << p.page_shift)) : 0;
            const auto prs = make_rsrc(pool + (((size_t)(ok ? pg : 0) * p.Hkv + j) << p.page_shift) * ROW,
                                       (uint32_t)nrows * ROW);
#pragma unroll
            for (int u = 0; u < NI; ++u)
                buffer_load_lds16(prs, dst + (wave * NI + u) * 1024, offs[u] + (k0 - prow0) * ROW, 0);
        }
    };

    // query operand of S^T, B layout, straight from memory: lane (n, g) of
    // step kk holds elements 32 kk + 8 g .. +7 of query tq + 16 qb + n
    // exactly as stored, so every product on the matrix cores is exact in
    // fp32; the scale log2(e)/sqrt(D) is applied to the fp32 scores.  Queries
    // past the prompt are zero.  The bias term b_q . k is the same for every
    // query of the head: over float caches the append computed it for every
    // key (p.bterm) and it seeds the scores' accumulators; over the INT8
    // staging it is computed here, with the bias as a second B operand (the
    // same in every column), and added to the scores in fp32.  The loads are
    // unconditional (a query past the prompt reads the last row, selected
    // away) so that they are all in flight together.
    u32x4 qraw[kQB][KK], braw[KK];
    if constexpr (BIAS && SC) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            braw[kk] = *(const u32x4*)((const uint16_t*)p.bias + (size_t)h * D + 32 * kk + 8 * g);
    }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const int tc = min(tq + 16 * qb + n, Sb - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qraw[qb][kk] = *(const u32x4*)((const uint16_t*)p.q + (((size_t)b * p.S + tc) * p.H + h) * D + 32 * kk + 8 * g);
    }
    issue(false, 0, ktile0, koffs, kscl0);
    issue(true, 0, vtile0, voffs, vscl0);
    issue(false, kPK, ktile1, koffs, kscl1);
    vec8 qv[kQB][KK], bv[KK];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const bool live = tq + 16 * qb + n < Sb;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qv[qb][kk] = MF::bits8(live ? qraw[qb][kk] : u32x4{0u, 0u, 0u, 0u});
    }
    if constexpr (BIAS && SC) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) bv[kk] = MF::bits8(braw[kk]);
    }
    const float c = p.qscale;               // log2(e) / sqrt(D)
    const float inv_c = 1.0f / c;

    // online softmax of query tq + 16 qb + n (the lane's column), in the
    // log2 domain (score x c).  m is the reference the weights are taken
    // against; it is raised only when some query of the wave sees a score
    // more than kLazy above its own, so a weight never exceeds 2^kLazy and
    // most steps skip the rescale of O (in exact arithmetic the result does
    // not depend on the reference).  thr is that bound in unscaled units.
    float m[kQB], l[kQB], thr[kQB];         // l: this lane's share of the sum
    f32x4 acc[kQB][DT];                     // O^T[16 tn + 4g + i][query tq + 16 qb + n]
    f32x4 lsum[kQB];                        // on the matrix cores: the sum for query tq + 16 qb + n
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        m[qb] = kNegInfP;
        thr[qb] = kNegInfP;
        l[qb] = 0.0f;
        lsum[qb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int tn = 0; tn < DT; ++tn) acc[qb][tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // per-lane LDS offsets: K row n of a 16-row block at step kk; V row
    // 4g + n/4 of a 16-row block, bytes 8 (n % 4) .. +7 of column tile tn
    // (the swizzles depend on the row only modulo 16)
    int koff[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) koff[kk] = n * ROW + (((4 * kk + g) ^ kswz(n)) * 16);
    const int vrow = 4 * g + (n >> 2);
    const int vsw = vswz(vrow);
    const int vbase = vrow * ROW + ((n & 3) >> 1) * 16 + (n & 1) * 8;

    // The keys go in steps of 32 (two per 64-key tile), software-pipelined
    // so that the matrix cores have work while the softmax runs: step j
    // takes the softmax of its scores S(j), then computes S(j + 1) = K Q^T
    // for the next step interleaved with the exponentials of step j, then
    // O^T += V^T P(j).  K tiles are needed one step before V tiles, so the
    // two are double-buffered a step apart: at every even step (new tile T)
    // the workgroup waits for V(T) and refills the other V buffer with
    // V(T + 1); at every odd step it waits for K(T + 1) and refills the other
    // K buffer with K(T + 2).  Each load has two steps to land, and LDS holds
    // two K and two V tiles.  Waves whose queries end earlier keep taking
    // part in the barriers and loads.
    const int nsteps = (kend + 31) / 32;
    const int last_j = tq < Sb ? tq / 32 : -1;   // this wave's last (diagonal) step
    // Every refill is issued, also past the last tile (its offsets lie past
    // the buffer's end, so it writes zeros into a buffer no step reads
    // again): the waits are then always "all but the newest batch of NI
    // loads", and neither they nor the loads sit behind a branch, whose join
    // made the compiler wait for every load in flight before the LDS reads.
    // s_waitcnt vmcnt(NI): the gfx9 encoding puts vmcnt in bits 3:0, expcnt
    // (7) in 6:4 and lgkmcnt (15) in 11:8; through the builtin the compiler
    // sees the wait too.
    constexpr int NBK = NI + (SC || kBiasTerms ? 1 : 0);   // loads per lane per K refill
    constexpr int NBV = NI + (SC ? 1 : 0);                 // loads per lane per V refill
    auto wait_one_batch_behind = [&](auto nb) { __builtin_amdgcn_s_waitcnt(0x0F70 | decltype(nb)::value); };
    // A workgroup barrier for LDS that leaves the newest tile loads in
    // flight (__syncthreads would wait for every load into LDS): this wave's
    // LDS accesses complete (lgkmcnt(0); vmcnt 63, expcnt 7 untouched), then
    // s_barrier, which the compiler may not move memory accesses across.
    auto lds_barrier = [&]() {
        __builtin_amdgcn_s_waitcnt(0xC07F);
        asm volatile("s_barrier" ::: "memory");
    };
    static_assert(NI == 1 || NI == 2 || NI == 4, "tile loads per lane");
    auto clear_v_tail = [&](int T, unsigned char* vt) {      // rows past kend of a partial tile
        if (T * kPK + kPK > kend) {
            for (int off = (kend - T * kPK) * ROW + tid * 16; off < TILE; off += 256 * 16)
                *(u32x4*)(vt + off) = u32x4{0u, 0u, 0u, 0u};
            lds_barrier();
        }
    };

    // unscaled S^T for the 32 keys `half` of the tile in K buffer kt: row =
    // key 32 half + 16 h2 + 4g + i, column = query tq + 16 qb + n.  Float
    // caches with a bias: the accumulators start from the keys' bias terms
    // (tbuf, the tile's term buffer), so the scores come out with b_q . k
    // added.  INT8 staging with a bias: entry kQB holds b_q . k (every column
    // alike).
    typedef f32x4 Scores[kQB + 1][2];
    auto qk = [&](Scores& sa, const unsigned char* kt, const unsigned char* tbuf, int half) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            f32x4 seed = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (kBiasTerms) seed = *(const f32x4*)((const float*)(tbuf + wave * 256) + 32 * half + 16 * h2 + 4 * g);
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) sa[qb][h2] = seed;
            sa[kQB][h2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const vec8 ka = MF::bits8(*(const u32x4*)(kt + (32 * half + 16 * h2) * ROW + koff[kk]));
#pragma unroll
                for (int qb = 0; qb < kQB; ++qb) sa[qb][h2] = MF::mma32(ka, qv[qb][kk], sa[qb][h2]);
                if constexpr (BIAS && SC) sa[kQB][h2] = MF::mma32(ka, bv[kk], sa[kQB][h2]);
            }
        }
    };

    // SC: the key's K scale goes on its raw score (bias term included) as
    // soon as the scores are complete, while K's scale buffer still holds
    // that tile (the odd step after refills it); slot kQB is then unused
    auto fold_k_scale = [&](Scores& sa, const unsigned char* sbuf, int half) {
        const float* ks = (const float*)(sbuf + wave * 256) + 32 * half + 4 * g;
        const f32x4 k0s = *(const f32x4*)ks, k1s = *(const f32x4*)(ks + 16);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa[qb][0][i] = (BIAS ? sa[qb][0][i] + sa[kQB][0][i] : sa[qb][0][i]) * k0s[i];
                sa[qb][1][i] = (BIAS ? sa[qb][1][i] + sa[kQB][1][i] : sa[qb][1][i]) * k1s[i];
            }
    };

    Scores scur, snext;
    __builtin_amdgcn_s_waitcnt(0x0F70);     // the first tiles (and the query) landed
    __syncthreads();
    clear_v_tail(0, vtile0);
    if (0 <= last_j) {
        qk(scur, ktile0, kscl0, 0);
        if constexpr (SC) fold_k_scale(scur, kscl0, 0);
    }

    // step j = j0 + U of a 4-step (two-tile) group: buffers by U
    auto step = [&](const int j0, auto U) {
        constexpr int u = decltype(U)::value;
        const int j = j0 + u;
        const int T = j / 2;
        unsigned char* const vt = (u / 2) ? vtile1 : vtile0;               // V(T)
        if constexpr (u % 2 == 0) {
            // new tile T: V(T) must have landed; V(T - 1)'s buffer is free
            if (j > 0) {
                wait_one_batch_behind(std::integral_constant<int, NBK>{});   // K(T + 1) was issued after V(T)
                lds_barrier();
                clear_v_tail(T, vt);
            }
            issue(true, T * kPK + kPK, (u / 2) ? vtile0 : vtile1, voffs, (u / 2) ? vscl0 : vscl1);
        } else {
            // K(T + 1) must have landed; K(T)'s buffer is free for K(T + 2)
            wait_one_batch_behind(std::integral_constant<int, NBV>{});   // V(T + 1) was issued after K(T + 1)
            lds_barrier();
            issue(false, T * kPK + 2 * kPK, (u / 2) ? ktile1 : ktile0, koffs, (u / 2) ? kscl1 : kscl0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j > last_j) return;
        const int kb = 32 * j;              // first key of the step
        // scores of this step; slot 4 h2 + i of this lane: key kb + 16 h2 + 4g + i
        float s[kQB][8];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s[qb][4 * h2 + i] = scur[qb][h2][i];
        if (j == last_j) {                  // the diagonal step: causal mask (also covers
                                            // keys past the prompt)
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (kb + 16 * (e / 4) + 4 * g + e % 4 > tq + 16 * qb + n) s[qb][e] = kNegInfP;
        }
        // the reference only needs raising when some score lies more than
        // kLazy above it; the maxima are taken only then
        bool raise = false;
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int e = 0; e < 8; ++e) raise = raise || s[qb][e] > thr[qb];
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                const float mt = fmaxf(fmaxf(fmaxf(s[qb][0], s[qb][1]), fmaxf(s[qb][2], s[qb][3])),
                                       fmaxf(fmaxf(s[qb][4], s[qb][5]), fmaxf(s[qb][6], s[qb][7])));
                const float mn = fmaxf(m[qb], column_max(mt) * c);
                const float alpha = fast_exp2(m[qb] - (mn == kNegInfP ? 0.0f : mn));
                m[qb] = mn;
                thr[qb] = (mn + kLazy) * inv_c;
                if constexpr (kSumOnMfma<KV, SC>) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) lsum[qb][i] *= alpha;
                } else {
                    l[qb] *= alpha;
                }
#pragma unroll
                for (int tn = 0; tn < DT; ++tn)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[qb][tn][i] *= alpha;
            }
        }
        // S(j + 1) for the next step (K of tile (j + 1) / 2), interleaved by
        // the scheduler with this step's exponentials.  Unconditional, so
        // that no branch separates the two: after a wave's last step the
        // result is not used (and may come from stale LDS).
        qk(snext, (u == 0 || u == 3) ? ktile0 : ktile1, (u == 0 || u == 3) ? kscl0 : kscl1, (j + 1) % 2);
        vec8 ph[kQB], pl[kQB];
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
            const float ms = m[qb] == kNegInfP ? 0.0f : m[qb];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s[qb][e] = fast_exp2(__builtin_fmaf(s[qb][e], c, -ms));
                if constexpr (!kSumOnMfma<KV, SC>) l[qb] += s[qb][e];
            }
            if constexpr (SC) {             // code x scale: the key's V scale on its weight
                const float* vs = (const float*)(((u / 2) ? vscl1 : vscl0) + wave * 256) + 32 * (j % 2) + 4 * g;
                const f32x4 v0s = *(const f32x4*)vs, v1s = *(const f32x4*)(vs + 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s[qb][i] *= v0s[i];
                    s[qb][4 + i] *= v1s[i];
                }
            }
            split_weights<KV, kWeightSplit<KV, SC>>(s[qb], ph[qb], pl[qb]);
        }
        // O^T += V^T P^T: A = V^T (row 16 tn + n, the slots' keys, read
        // down V's columns), B = P^T (this lane's slots for its query)
#pragma unroll
        for (int tn = 0; tn < DT; ++tn) {
            const unsigned char* va0 = vt + 32 * (j % 2) * ROW + vbase + ((2 * tn) ^ vsw) * 16;
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(va0));
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(va0 + 16 * ROW));
            const vec8 va = __builtin_bit_cast(vec8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) {
                acc[qb][tn] = MF::mma32(va, ph[qb], acc[qb][tn]);
                if constexpr (kWeightSplit<KV, SC>) acc[qb][tn] = MF::mma32(va, pl[qb], acc[qb][tn]);
            }
        }
        if constexpr (kSumOnMfma<KV, SC>) {
            vec8 ones;
#pragma unroll
            for (int i = 0; i < 8; ++i) ones[i] = (_Float16)1.0f;
#pragma unroll
            for (int qb = 0; qb < kQB; ++qb) lsum[qb] = MF::mma32(ones, ph[qb], lsum[qb]);
        }
        if constexpr (SC) fold_k_scale(snext, (u == 0 || u == 3) ? kscl0 : kscl1, (j + 1) % 2);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) scur[qb][h2] = snext[qb][h2];
    };
    for (int j0 = 0; j0 < nsteps; j0 += 4) {
        step(j0, std::integral_constant<int, 0>{});
        if (j0 + 1 < nsteps) step(j0, std::integral_constant<int, 1>{});
        if (j0 + 2 < nsteps) step(j0, std::integral_constant<int, 2>{});
        if (j0 + 3 < nsteps) step(j0, std::integral_constant<int, 3>{});
    }
    // the last refills are still in flight: let them land before the wave
    // can end and the workgroup's LDS be handed on
    __builtin_amdgcn_s_waitcnt(0x0F70);

    // out[query][16 tn + 4g + i] = O^T / l, four consecutive columns
    // (8 bytes) per lane and tile
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
        const float inv = 1.0f / (kSumOnMfma<KV, SC> ? lsum[qb][0] : column_sum(l[qb]));
        const int t = tq + 16 * qb + n;
        if (t < Sb) {
            uint16_t* orow = (uint16_t*)p.out + (((size_t)b * p.S + t) * p.H + h) * D + 4 * g;
#pragma unroll
            for (int tn = 0; tn < DT; ++tn) {
                uint32_t hb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = acc[qb][tn][i] * inv;
                    hb[i] = KV == KV_F16 ? float_to_half_bits(v) : float_to_bf16_bits(v);
                }
                *(u32x2*)(orow + tn * 16) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
            }
        }
    }
}

template <int KV, int D>
hipError_t launch_append_t(const PrefillParams& p, hipStream_t s) {
    constexpr int RPB = 256 / (D / 8);
    const dim3 grid((unsigned)((p.S + RPB - 1) / RPB * p.Hkv), (unsigned)p.B);
    if (p.block_table)
        hipLaunchKernelGGL((prefill_append_kernel<KV, D, true>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_append_kernel<KV, D, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int KV, int D>
hipError_t launch_attention_t(const PrefillParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.B * p.H), (p.S + kPQ - 1) / kPQ);
    if (p.block_table) {
        if (p.bias) hipLaunchKernelGGL((prefill_attn_kernel<KV, D, true, true, false>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((prefill_attn_kernel<KV, D, true, false, false>), grid, dim3(256), 0, s, p);
    } else {
        if (p.bias) hipLaunchKernelGGL((prefill_attn_kernel<KV, D, false, true, false>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((prefill_attn_kernel<KV, D, false, false, false>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_append_i8_t(const PrefillParams& p, hipStream_t s) {
    constexpr int RPB = 256 / (D / 16);
    const dim3 grid((unsigned)((p.S + RPB - 1) / RPB * p.Hkv), (unsigned)p.B);
    if (p.block_table)
        hipLaunchKernelGGL((prefill_append_i8_kernel<D, true>), grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((prefill_append_i8_kernel<D, false>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

// the attention over the INT8 staging: contiguous rows of S positions,
// fp16 codes with per-key scales
template <int D>
hipError_t launch_attention_i8_t(const PrefillParams& p0, hipStream_t s) {
    PrefillParams p = p0;
    p.k_cache = p.stage_k;
    p.v_cache = p.stage_v;
    p.Lmax = p.S;                           // block_table stays: the page check
    const dim3 grid((unsigned)(p.B * p.H), (p.S + kPQ - 1) / kPQ);
    if (p.bias) hipLaunchKernelGGL((prefill_attn_kernel<KV_F16, D, false, true, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((prefill_attn_kernel<KV_F16, D, false, false, true>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_append_i8(const PrefillParams& p, int head_dim, hipStream_t s) {
    return head_dim == 64 ? launch_append_i8_t<64>(p, s) : launch_append_i8_t<128>(p, s);
}

hipError_t launch_prefill_attention_i8(const PrefillParams& p, int head_dim, hipStream_t s) {
    return head_dim == 64 ? launch_attention_i8_t<64>(p, s) : launch_attention_i8_t<128>(p, s);
}

hipError_t launch_prefill_append(const PrefillParams& p, int kv, int head_dim, hipStream_t s) {
    if (kv == KV_F16) return head_dim == 64 ? launch_append_t<KV_F16, 64>(p, s) : launch_append_t<KV_F16, 128>(p, s);
    if (kv == KV_BF16) return head_dim == 64 ? launch_append_t<KV_BF16, 64>(p, s) : launch_append_t<KV_BF16, 128>(p, s);
    return hipErrorInvalidValue;
}

hipError_t launch_prefill_attention(const PrefillParams& p, int kv, int head_dim, hipStream_t s) {
    if (kv == KV_F16)
        return head_dim == 64 ? launch_attention_t<KV_F16, 64>(p, s) : launch_attention_t<KV_F16, 128>(p, s);
    if (kv == KV_BF16)
        return head_dim == 64 ? launch_attention_t<KV_BF16, 64>(p, s) : launch_attention_t<KV_BF16, 128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace ftm
