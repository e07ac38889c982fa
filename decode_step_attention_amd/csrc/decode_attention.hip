// decode_attention.hip -- gfx950 kernels for one decode step of masked
// multi-head attention over a [B, Hkv, Lmax, D] KV cache.
//
// attention_kernel: one workgroup (4 wave64) owns one (sequence b, KV head j,
//   query-head group, chunk of positions).  It folds the QKV bias into the
//   query, streams the chunk's K and V rows once from HBM as 16-byte
//   vectors through buffer loads (rows past the valid range read as zero
//   and fetch nothing), reduces each q.k across the lanes holding one row
//   with DPP, keeps an online softmax state per row slot, and merges slots
//   and waves at the end.  The workgroup whose chunk holds the new position
//   appends the biased K/V row (fp32 add, RNE rounding or INT8 quantising)
//   and feeds it to the softmax from registers.  With one chunk per
//   sequence it writes the output; otherwise it writes the chunk's
//   (max, sum, unnormalised output) for the combine kernel.
// combine_kernel: merges the chunks' softmax states per (b, h).
//
// The method: fused decode attention with the new K/V appended to a
// pre-allocated cache ([lpnh.cn/news/2765398] sections 2.1 and 2.2), the
// maximum subtracted before exponentiation ([lpnh.cn/news/2765398] section
// 6.1), blockwise softmax statistics so a long sequence can be split into
// independent pieces ([pptc.cn/news/144085] section 2.2), grouped KV heads
// ([pptc.cn/news/144085] section 3.4) and an INT8 cache converted back at
// compute time ([pptc.cn/news/144085] section 3.1; [intelliparadigm.com
// .../2131745] section 2.1).  Scores never leave registers.
#include <algorithm>
#include <cstdio>
#include <cstdlib>

#include <map>
#include <mutex>

#include "gfx950.hpp"

// Scratch memory of the allocation-free decode call (ftm_decode_mha_static):
// each GPU the library runs on holds one copy until the process ends.  Host
// code never passes this name to a kernel: in host code it is only a
// stand-in, and the device address comes from hipGetSymbolAddress (see
// ftm::static_scratch below).
static __device__ __align__(256) unsigned char scratch[ftm::kStaticScratchBytes];

namespace ftm {
namespace {

constexpr int kWaves = 4;                 // waves per combine workgroup
constexpr int kThreads = 64 * kWaves;
// Cache policy of the K/V stream: non-temporal (every byte is used once).
constexpr int kStream = 2;
constexpr float kNegInf = -__builtin_inff();

// Cache element type: size and how a 16-byte vector unpacks into fp32.
template <int KV> struct Elem;
template <> struct Elem<KV_F32> {
    static constexpr int bytes = 4;
    __device__ static void unpack(const u32x4 w, float* x) {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
};
template <> struct Elem<KV_F16> {
    static constexpr int bytes = 2;
    __device__ static void unpack(const u32x4 w, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = half_bits_to_float(w[i] & 0xffffu);
            x[2 * i + 1] = half_bits_to_float(w[i] >> 16);
        }
    }
};
template <> struct Elem<KV_BF16> {
    static constexpr int bytes = 2;
    __device__ static void unpack(const u32x4 w, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Elem<KV_I8> {
    static constexpr int bytes = 1;
    // INT8 codes as fp32 (the scale is applied to the reduced dot product
    // and to the softmax weight, so it is not multiplied in here).
    __device__ static void unpack(const u32x4 w, float* x) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 4; ++k) x[4 * i + k] = (float)(int8_t)((w[i] >> (8 * k)) & 0xffu);
    }
};

// Activation type (q, k_new, v_new, bias, out): the cache type for float
// caches and fp16 next to an INT8 cache.
template <int KV> struct Act;
template <> struct Act<KV_F32> {
    __device__ static float ld(const void* p, size_t i) { return ((const float*)p)[i]; }
    __device__ static void st(void* p, size_t i, float v) { ((float*)p)[i] = v; }
};
template <> struct Act<KV_F16> {
    __device__ static float ld(const void* p, size_t i) { return half_bits_to_float(((const uint16_t*)p)[i]); }
    __device__ static void st(void* p, size_t i, float v) { ((uint16_t*)p)[i] = (uint16_t)float_to_half_bits(v); }
};
template <> struct Act<KV_BF16> {
    __device__ static float ld(const void* p, size_t i) { return bf16_bits_to_float(((const uint16_t*)p)[i]); }
    __device__ static void st(void* p, size_t i, float v) { ((uint16_t*)p)[i] = (uint16_t)float_to_bf16_bits(v); }
};
template <> struct Act<KV_I8> : Act<KV_F16> {};

// N consecutive activation elements starting at element `off` of `base`, as
// fp32, read as 16-byte vectors (rows of q, k_new, v_new and the bias are
// 16-byte aligned: D * element size is a multiple of 16 and the pointers
// are checked on the host).
template <int KV, int N>
__device__ __forceinline__ void load_act(const void* base, size_t off, float* x) {
    if constexpr (KV == KV_F32) {
        static_assert(N % 4 == 0, "");
        const u32x4* v = (const u32x4*)((const float*)base + off);
#pragma unroll
        for (int i = 0; i < N / 4; ++i) Elem<KV_F32>::unpack(v[i], x + 4 * i);
    } else {
        static_assert(N % 8 == 0, "");
        const u32x4* v = (const u32x4*)((const uint16_t*)base + off);
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            if constexpr (KV == KV_BF16) Elem<KV_BF16>::unpack(v[i], x + 8 * i);
            else Elem<KV_F16>::unpack(v[i], x + 8 * i);
        }
    }
}

template <int LPR> __device__ __forceinline__ float group_max(float v) {
    v = fmaxf(v, dpp<kQuadSwap1>(v));
    v = fmaxf(v, dpp<kQuadSwap2>(v));
    if constexpr (LPR == 8) v = fmaxf(v, dpp<kRowHalfMirror>(v));
    if constexpr (LPR >= 16) {
        v = fmaxf(v, dpp<kRowRor4>(v));
        v = fmaxf(v, dpp<kRowRor8>(v));
    }
    if constexpr (LPR == 32) v = fmaxf(v, __shfl_xor(v, 16));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off));
    return v;
}
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}


// Paged cache: position `pos` of (sequence b, KV head j) is row pos mod P of
// page tbl[pos / P] of a [n_pages, Hkv, P, row] pool (P a power of two; tbl
// is sequence b's block-table row).  Descriptor starting at the row of
// `pos` (wave-uniform) and covering the rows of its page that lie below
// `end`: empty when pos >= end, zeros and `bad` set when the table names a
// page outside the pool.  Branch-free: the table index is clamped to the
// last page below `end`, so the entry read always lies in the row.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* pool, int row_bytes,
                                                            const int32_t* tbl, const Params& p,
                                                            int j, int pos, int end, bool& bad) {
    const int sh = p.page_shift;
    const int idx = min(pos >> sh, max(end - 1, 0) >> sh);
    // the table is never written by a kernel: read it as constant memory,
    // through the scalar cache, so that the read does not queue behind the
    // K/V loads in flight
    const int page = ((const __attribute__((address_space(4))) int32_t*)tbl)[idx];
    const int in_page = pos & ((1 << sh) - 1);
    const bool valid = (unsigned)page < (unsigned)p.n_pages;
    int rows = min(end - pos, (1 << sh) - in_page);
    rows = rows > 0 ? rows : 0;
    bad |= rows > 0 && !valid;
    rows = valid ? rows : 0;
    const size_t row = (((size_t)(valid ? page : 0) * p.Hkv + j) << sh) + in_page;
    return make_rsrc((const char*)pool + row * row_bytes, (uint32_t)rows * (uint32_t)row_bytes);
}

// Where the appended row of (b, j) at position pnew lives: its row index in
// the cache (or pool) and the element offset of the V plane of the INT8
// scales.  Paged: false when the table names a page outside the pool.
template <bool PG>
__device__ __forceinline__ bool new_row_index(const Params& p, int b, int j, int pnew, size_t& row,
                                              size_t& scale_plane) {
    if constexpr (PG) {
        const int page = p.block_table[(size_t)b * p.max_pages + (pnew >> p.page_shift)];
        row = (((size_t)page * p.Hkv + j) << p.page_shift) + (pnew & ((1 << p.page_shift) - 1));
        scale_plane = ((size_t)p.n_pages * p.Hkv) << p.page_shift;
        return (unsigned)page < (unsigned)p.n_pages;
    } else {
        row = ((size_t)b * p.Hkv + j) * p.Lmax + pnew;
        scale_plane = (size_t)p.B * p.Hkv * p.Lmax;
        return true;
    }
}

// ---------------------------------------------------------------------------
// The new row: x = fl32(new + bias), stored as the cache type.  `stored`
// receives what the cache now holds, as fp32 (INT8: the code), `scale` the
// INT8 scale (1 otherwise), `packed` the 16 bytes this lane writes.
// ---------------------------------------------------------------------------
template <int KV, int EPL, int LPR>
__device__ __forceinline__ void store_new_row(float* x, float* stored, float& scale, u32x4& packed);

template <int KV, int D, int EPL, int LPR>
__device__ __forceinline__ void make_new_row(const Params& p, const void* src, int bias_row,
                                             size_t src_row, int c, float* stored, float& scale,
                                             u32x4& packed) {
    float x[EPL];
    load_act<KV, EPL>(src, src_row * D + c * EPL, x);
    if (p.bias) {
        float bx[EPL];
        load_act<KV, EPL>(p.bias, (size_t)bias_row * D + c * EPL, bx);
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = x[e] + bx[e];   // one fp32 rounding
    }
    store_new_row<KV, EPL, LPR>(x, stored, scale, packed);
}

// x (the biased row slice, fp32) as the cache type: `stored` what the cache
// will hold, as fp32 (INT8: the code), `scale` the INT8 scale (1 otherwise),
// `packed` the 16 bytes to write.
template <int KV, int EPL, int LPR>
__device__ __forceinline__ void store_new_row(float* x, float* stored, float& scale, u32x4& packed) {
    scale = 1.0f;
    if constexpr (KV == KV_F32) {
        packed = u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                       __float_as_uint(x[3])};
#pragma unroll
        for (int e = 0; e < EPL; ++e) stored[e] = x[e];
    } else if constexpr (KV == KV_F16 || KV == KV_BF16) {
        uint32_t hb[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            hb[e] = KV == KV_F16 ? float_to_half_bits(x[e]) : float_to_bf16_bits(x[e]);
            stored[e] = KV == KV_F16 ? half_bits_to_float(hb[e]) : bf16_bits_to_float(hb[e]);
        }
        packed = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16),
                       hb[6] | (hb[7] << 16)};
    } else {
        // symmetric INT8: s = absmax / 127 (IEEE division), code = rint(x / s)
        // clamped to [-127, 127]; a zero row keeps s = 0 and zero codes.
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
        amax = group_max<LPR>(amax);
        scale = amax / 127.0f;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            float q = 0.0f;
            if (scale != 0.0f) q = fminf(fmaxf(rintf(x[e] / scale), -127.0f), 127.0f);
            stored[e] = q;
            w[e / 4] |= ((uint32_t)(int32_t)q & 0xffu) << (8 * (e % 4));
        }
        packed = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// ---------------------------------------------------------------------------
// Attention pass.  Template: cache type, head dim, query heads per pass (GT),
// 16-byte loads per lane per K/V stream per iteration (U), waves per
// workgroup (NW).
//
// Each wave streams its own rows with a software pipeline at half-iteration
// granularity: while the softmax and P.V of iteration i run, the K loads of
// iteration i+1 are already in flight, and the V loads of i+1 go out as soon
// as P.V of i has consumed its registers.  Loads past the valid range are
// clipped by the buffer descriptor (they return zeros and fetch nothing), so
// the prefetch after the last iteration costs issue slots only.
// ---------------------------------------------------------------------------
// PG: paged cache; LP (paged only): a page holds at least the rows one wave
// loads per iteration, so one table read and one descriptor per stream serve
// them all.
template <int KV, int D, int GT, int U, int NW, bool PG, bool LP>
__global__ void __launch_bounds__(64 * NW) attention_kernel(const Params p) {
    using E = Elem<KV>;
    using A = Act<KV>;
    constexpr int NT = 64 * NW;
    constexpr int EPL = 16 / E::bytes;      // elements per lane per load
    constexpr int LPR = D / EPL;            // lanes per cache row
    constexpr int RPI = 64 / LPR;           // rows per wave-wide load
    constexpr int ROW_BYTES = D * E::bytes;
    constexpr int WAVE_ROWS = RPI * U;      // rows per wave per iteration
    constexpr int BLOCK_ROWS = NW * WAVE_ROWS;
    constexpr bool I8 = KV == KV_I8;
    static_assert(LPR >= 4 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row must span 4..32 lanes");

    __shared__ float sm_m[NW][GT];
    __shared__ float sm_l[NW][GT];
    __shared__ float sm_o[NW][GT][D];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane / LPR;               // row slot of this lane
    const int c = lane % LPR;               // 16-byte column slice of the row
    const int chunk = blockIdx.x;
    const int j = blockIdx.y / p.n_hg;
    const int hgi = blockIdx.y - j * p.n_hg;
    const int b = blockIdx.z;
    const int h0 = j * p.G + hgi * GT;
    const int heads_here = min(GT, p.G - hgi * GT);
    // the length is the same for the whole workgroup; say so, so that the
    // buffer descriptors built from it live in scalar registers
    const int L = __builtin_amdgcn_readfirstlane(p.seq_lens ? p.seq_lens[b] : p.step);

    if (L < 1 || L > p.step) {              // invalid length: NaN rows, no append
        if (p.direct && chunk == 0)
            for (int idx = threadIdx.x; idx < GT * D; idx += NT)
                if (idx / D < heads_here)
                    A::st(p.out, ((size_t)b * p.H + h0 + idx / D) * D + idx % D, __builtin_nanf(""));
        return;
    }
    const int n_chunks = (L + p.chunk - 1) / p.chunk;
    if (chunk >= n_chunks) return;
    const int c0 = chunk * p.chunk;
    const int c1 = min(c0 + p.chunk, L);
    const int stream_end = min(c1, L - 1);  // the new row L-1 comes from registers
    const bool owns_new = c1 == L;

    // contiguous cache: one descriptor per stream over rows [0, stream_end)
    // of this (b, j); paged: one per page, built where the rows are loaded
    const size_t row0 = ((size_t)b * p.Hkv + j) * p.Lmax;   // contiguous: row 0 of this (b, j)
    const uint32_t valid_bytes = PG ? 0u : (uint32_t)max(stream_end, 0) * ROW_BYTES;
    const auto krs = make_rsrc(PG ? nullptr : (const char*)p.k_cache + row0 * ROW_BYTES, valid_bytes);
    const auto vrs = make_rsrc(PG ? nullptr : (const char*)p.v_cache + row0 * ROW_BYTES, valid_bytes);
    const size_t plane = PG ? ((size_t)p.n_pages * p.Hkv) << p.page_shift
                            : (size_t)p.B * p.Hkv * p.Lmax;  // INT8 scale plane
    const bool flat_i8 = I8 && !PG;
    const auto ksrs = make_rsrc(flat_i8 ? p.kv_scales + row0 : nullptr, flat_i8 ? max(stream_end, 0) * 4 : 0);
    const auto vsrs = make_rsrc(flat_i8 ? p.kv_scales + plane + row0 : nullptr, flat_i8 ? max(stream_end, 0) * 4 : 0);
    const int32_t* tbl = PG ? p.block_table + (size_t)b * p.max_pages : nullptr;
    bool bad = false;                       // paged: the table named a page outside the pool

    u32x4 kr[U], vr[U];
    // INT8 scales, contiguous cache: the WAVE_ROWS scales of an iteration
    // are contiguous, so lane l loads the scale of row l (one coalesced load
    // per 64 rows) and the lanes holding a row fetch it with a cross-lane
    // read at use.  Paged: the lanes of a row load its scale from the row's
    // page, one load per RPI rows.
    constexpr int NS = PG ? U : (WAVE_ROWS + 63) / 64;
    float ks_all[NS], vs_all[NS];
    // lanes past the iteration's rows point outside the descriptor: no fetch
    auto scale_off = [&](int base, int i) {
        return i * 64 + lane < WAVE_ROWS ? (base + i * 64 + lane) * 4 : 0x7fffffff;
    };
    // rows base + u*RPI .. + RPI-1 lie in one page (P >= 16 >= RPI, both
    // powers of two, base a multiple of RPI); with LP so do all WAVE_ROWS
    // rows from base (P >= WAVE_ROWS, base a multiple of WAVE_ROWS)
    auto issue_stream = [&](const void* pool, const __amdgpu_buffer_rsrc_t& rs,
                            const __amdgpu_buffer_rsrc_t& srs, size_t splane, u32x4* dst,
                            float* sdst, int base) {
        if constexpr (PG && LP) {
            const auto prs = page_rsrc(pool, ROW_BYTES, tbl, p, j, base, stream_end, bad);
#pragma unroll
            for (int u = 0; u < U; ++u)
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(prs, (u * RPI + r) * ROW_BYTES + c * 16, 0, kStream);
            if constexpr (I8) {
                const auto pss = page_rsrc(p.kv_scales + splane, 4, tbl, p, j, base, stream_end, bad);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    sdst[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pss, (u * RPI + r) * 4, 0, kStream));
            }
        } else if constexpr (PG) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int pos = base + u * RPI;
                const auto prs = page_rsrc(pool, ROW_BYTES, tbl, p, j, pos, stream_end, bad);
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(prs, r * ROW_BYTES + c * 16, 0, kStream);
                if constexpr (I8) {
                    const auto pss = page_rsrc(p.kv_scales + splane, 4, tbl, p, j, pos, stream_end, bad);
                    sdst[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pss, r * 4, 0, kStream));
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
                dst[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (base + u * RPI + r) * ROW_BYTES + c * 16, 0, kStream);
            if constexpr (I8) {
#pragma unroll
                for (int i = 0; i < NS; ++i)
                    sdst[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(srs, scale_off(base, i), 0, kStream));
            }
        }
    };
    auto issue_k = [&](int base) { issue_stream(p.k_cache, krs, ksrs, 0, kr, ks_all, base); };
    auto issue_v = [&](int base) { issue_stream(p.v_cache, vrs, vsrs, plane, vr, vs_all, base); };
    // scale of row u*RPI + r of this iteration (64 is a multiple of RPI)
    auto row_scale = [&](const float* all, int u) {
        if constexpr (PG) return all[u];
        else return __shfl(all[(u * RPI) / 64], (u * RPI) % 64 + r);
    };

    // the first K/V loads go out before the query is read, so their latency
    // and the query's overlap
    int base = c0 + wave * WAVE_ROWS;
    issue_k(base);
    issue_v(base);
    __builtin_amdgcn_sched_barrier(0);

    // query with bias, in fp32, pre-scaled by log2(e)/sqrt(D) so the softmax
    // runs on exp2 (heads past the group read a valid row and are zeroed)
    float qv[GT][EPL];
#pragma unroll
    for (int g = 0; g < GT; ++g)
        load_act<KV, EPL>(p.q, ((size_t)b * p.H + min(h0 + g, p.H - 1)) * D + c * EPL, qv[g]);
    if (p.bias) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float bx[EPL];
            load_act<KV, EPL>(p.bias, (size_t)min(h0 + g, p.H - 1) * D + c * EPL, bx);
#pragma unroll
            for (int e = 0; e < EPL; ++e) qv[g][e] = qv[g][e] + bx[e];
        }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[g][e] = g < heads_here ? qv[g][e] * p.qscale : 0.0f;

    float m[GT], l[GT], o[GT][EPL];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = 0.0f;
    }

    for (; base < stream_end; base += BLOCK_ROWS) {
        // scores (log2 domain) from this iteration's K
        float s[GT][U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[EPL];
            E::unpack(kr[u], x);
            const bool valid = base + u * RPI + r < stream_end;
            float ksu = 1.0f;
            if constexpr (I8) ksu = row_scale(ks_all, u);
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                float d = 0.0f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) d = fmaf(qv[g][e], x[e], d);
                d = group_sum<LPR>(d);
                if constexpr (I8) d *= ksu;
                s[g][u] = valid ? d : kNegInf;
            }
        }
        // K registers are free: next iteration's K goes out now
        __builtin_amdgcn_sched_barrier(0);
        issue_k(base + BLOCK_ROWS);
        __builtin_amdgcn_sched_barrier(0);
        // online softmax: new running max, rescale, weights
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float mt = s[g][0];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[g][u]);
            const float mn = fmaxf(m[g], mt);
            const float ms = mn == kNegInf ? 0.0f : mn;
            const float a = fast_exp2(m[g] - ms);
            l[g] *= a;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[g][e] *= a;
            m[g] = mn;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                s[g][u] = fast_exp2(s[g][u] - ms);
                l[g] += s[g][u];
            }
        }
        // weighted sum of V
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[EPL];
            E::unpack(vr[u], x);
            float vsu = 1.0f;
            if constexpr (I8) vsu = row_scale(vs_all, u);
#pragma unroll
            for (int g = 0; g < GT; ++g) {
                float w = s[g][u];
                if constexpr (I8) w *= vsu;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(w, x[e], o[g][e]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_v(base + BLOCK_ROWS);
        __builtin_amdgcn_sched_barrier(0);
    }

    // append the new row and add it to the softmax of row slot 0 of wave 0
    // (after the stream: a load issued while the CU's loads are in flight
    // waits behind them, and wave 0 waiting for the row at the start
    // measured slower, 7b 43.9 against 43.0 us and int8 425 against 416 us)
    if (owns_new && wave == 0) {
        const int pnew = L - 1;
        const size_t src_row = (size_t)b * p.Hkv + j;
        float kx[EPL], vx[EPL], ks, vs;
        u32x4 kpk, vpk;
        make_new_row<KV, D, EPL, LPR>(p, p.k_new, p.H + j, src_row, c, kx, ks, kpk);
        make_new_row<KV, D, EPL, LPR>(p, p.v_new, p.H + p.Hkv + j, src_row, c, vx, vs, vpk);
        size_t nrow, splane;
        const bool ok = new_row_index<PG>(p, b, j, pnew, nrow, splane);
        if (!ok) bad = true;
        if (ok && hgi == 0 && r == 0) {
            *(u32x4*)((char*)p.k_cache + nrow * ROW_BYTES + c * 16) = kpk;
            *(u32x4*)((char*)p.v_cache + nrow * ROW_BYTES + c * 16) = vpk;
            if constexpr (I8) {
                if (c == 0) {
                    p.kv_scales[nrow] = ks;
                    p.kv_scales[splane + nrow] = vs;
                }
            }
        }
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(qv[g][e], kx[e], d);
            d = group_sum<LPR>(d);
            if constexpr (I8) d *= ks;
            if (r == 0) {
                const float mn = fmaxf(m[g], d);
                const float a = fast_exp2(m[g] - mn);
                const float w = fast_exp2(d - mn);
                l[g] = l[g] * a + w;
                const float wv = I8 ? w * vs : w;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(wv, vx[e], o[g][e] * a);
                m[g] = mn;
            }
        }
    }

    // a page outside the pool makes the result NaN (the sum carries it
    // through every merge)
    if (bad) {
#pragma unroll
        for (int g = 0; g < GT; ++g) l[g] = __builtin_nanf("");
    }

    // merge the row slots of each wave
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
            const float m2 = __shfl_xor(m[g], off);
            const float l2 = __shfl_xor(l[g], off);
            const float mn = fmaxf(m[g], m2);
            const float ms = mn == kNegInf ? 0.0f : mn;
            const float a1 = fast_exp2(m[g] - ms);
            const float a2 = fast_exp2(m2 - ms);
            l[g] = l[g] * a1 + l2 * a2;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[g][e] = o[g][e] * a1 + __shfl_xor(o[g][e], off) * a2;
            m[g] = mn;
        }
    }
    if (r == 0) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_o[wave][g][c * EPL + e] = o[g][e];
            if (c == 0) {
                sm_m[wave][g] = m[g];
                sm_l[wave][g] = l[g];
            }
        }
    }
    __syncthreads();

    // merge the waves and write
    for (int idx = threadIdx.x; idx < GT * D; idx += NT) {
        const int g = idx / D;
        const int d = idx - g * D;
        if (g >= heads_here) continue;
        float M = sm_m[0][g];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
        const float ms = M == kNegInf ? 0.0f : M;
        float lsum = 0.0f, acc = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float a = fast_exp2(sm_m[w][g] - ms);
            lsum += a * sm_l[w][g];
            acc += a * sm_o[w][g][d];
        }
        const size_t bh = (size_t)b * p.H + h0 + g;
        if (p.direct) {
            A::st(p.out, bh * D + d, acc / lsum);
        } else {
            p.ws_o[(bh * p.S + chunk) * D + d] = acc;
            if (d == 0) {
                p.ws_ml[(bh * p.S + chunk) * 2] = M;
                p.ws_ml[(bh * p.S + chunk) * 2 + 1] = lsum;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped-query pass on the matrix cores, for fp16/bf16 caches with 4 or 8
// query heads per KV head.  Both products are small dense contractions and
// run as MFMA, heads padded to 16:
//  * S^T = K . Q^T with v_mfma_f32_16x16x32: each lane's 16-byte slice of a
//    K row is its A operand as loaded (no conversion, no cross-lane sum).
//    The fp32 query (bias added, log2(e)/sqrt(D) folded in) is the B
//    operand as two halves, hi = round(q) and lo = round(q - hi), whose
//    products accumulate in fp32: about 16 (bf16) or 22 (fp16) bits of q.
//  * O += P . V with v_mfma_f32_16x16x16: S^T leaves each lane holding four
//    consecutive positions of one head, which is exactly the A-operand
//    layout of P, so the weights need no shuffle; they enter as hi/lo
//    halves too.  V must be read down its columns, so every V tile goes
//    through a per-wave LDS buffer whose row pitch (D*2 + 8 bytes) puts the
//    four rows one operand reads on distinct banks.
// The softmax runs on the S^T tile: lane (g, n) holds head n at positions
// 4g..4g+3 of each 16-position tile.
// ---------------------------------------------------------------------------
// Device-coherent accesses for data handed between workgroups on different
// XCDs (relaxed atomics at agent scope: written through to, and read from,
// the device coherence point).
__device__ __forceinline__ void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's stores have been acknowledged.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-position tiles whose loads each wave of the grouped-query pass keeps
// in flight (register sets in rotation).
constexpr int kGqaDepth = 2;

// Largest batch the range schedule handles (each lane of a wave holds up to
// four sequences' lengths); larger batches take the vector-ALU pass.
constexpr int kGqaMaxBatch = 256;

// LDS layout of the grouped-query pass, per wave: a K tile and a V tile of
// 16 positions, row pitches chosen so that the operand reads hit distinct
// banks: K rows are read 16 B at a time across 16 rows (pitch = row + 16 B),
// V is read down its columns by the transposing read, 4 rows x 32 B per
// 16-lane group (pitch = row + 32 B).  The query operand (hi and lo halves
// for 16 padded heads) is shared by the workgroup, with the K pitch.
template <int D> struct GqaLds {
    static constexpr int ROW = D * 2;
    static constexpr int KPITCH = ROW + 16;
    static constexpr int VPITCH = ROW + 32;
    static constexpr int WAVE = 16 * KPITCH + 16 * VPITCH;
    static constexpr int QBYTES = 2 * 16 * KPITCH;
};

// Segments one workgroup streams together, each wave moving from one to the
// next on its own, with no barrier between them.
constexpr int kGqaMaxSeg = 2;

// One segment: positions [pos0, pos1) of unit (b, j, hgi) of length L.
struct GqaSeg {
    int b, j, hgi, L, pos0, pos1;
};

// Streams up to kGqaMaxSeg segments with the whole workgroup.  Each wave
// takes a fixed share of the segments' 16-position tiles, in order, with
// its K/V loads running DEPTH tiles ahead across the segment boundary and
// one softmax state per segment in registers; a wave that reaches the next
// segment starts on it at once.  At the end, per segment, the waves' states
// and the appended row's (when the segment holds it) are merged through LDS
// into `out` (a whole unit) or the piece's partial slot.
template <int KV, int D, int HP, int NW, bool PG>
__device__ __forceinline__ void gqa_group(const Params& p, unsigned char* tiles, unsigned char* qbufs,
                                          float (*sm_m)[NW][HP], float (*sm_l)[NW][HP], float (*sm_nm)[HP],
                                          float (*sm_nl)[HP], float* sm_newo,
                                          const GqaSeg (&sg)[kGqaMaxSeg], const int (&npieces)[kGqaMaxSeg],
                                          int nseg, int blk, bool first_group) {
    using MF = Mfma<KV>;
    using LD = GqaLds<D>;
    using A = Act<KV>;
    typedef typename MF::vec8 vec8;
    typedef typename MF::vec4 vec4;
    constexpr int S = kGqaMaxSeg;
    constexpr int NTH = 64 * NW;
    constexpr int ROW_BYTES = D * 2;
    constexpr int KK = D / 32;              // S^T: MFMA steps over the head dim
    constexpr int DT = D / 16;              // O: 16-column tiles
    constexpr int EPL = 8;                  // loads: elements per lane
    constexpr int LPR = D / EPL;            // loads: lanes per row
    constexpr int RPI = 64 / LPR;           // loads: rows per wave-wide load
    constexpr int VL = 16 / RPI;            // loads per 16-position tile, each of K and V
    constexpr int DEPTH = kGqaDepth;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;                // MFMA layout: k-slot group, position quad
    const int n = lane & 15;                // MFMA layout: K row / head column / V column
    const int r = lane / LPR;               // load layout: row slot
    const int c = lane % LPR;               // load layout: 16-byte column slice
    unsigned char* ktile = tiles + wave * LD::WAVE;
    unsigned char* vtile = ktile + 16 * LD::KPITCH;

    // The group's tiles: segment 0's 16-position tiles, then segment 1's,
    // numbered 0 .. ntot - 1, dealt out in rounds of 4 (A + B) tiles: each
    // of the four older waves (the first wave on each SIMD, which the SIMD
    // serves first) takes A consecutive tiles of a round, each younger wave
    // B.  A wave goes through its tiles in order, across the segment
    // boundary without a pause.  A fixed assignment: every call sums the
    // same positions in the same order (the results do not depend on
    // timing).  Per segment: the streamed end (the appended row is handled
    // apart), its tiles, and the descriptor inputs: contiguous, one
    // descriptor per stream over rows [0, end) of the unit; paged, one per
    // tile (tiles never straddle a page, P >= 16).
    static_assert(S == 2, "the tile numbering covers two segments");
    int send[S], ntl[S];
    size_t row0[S];                         // contiguous: the unit's first cache row
    const int32_t* tbl[S];                  // paged: the sequence's block-table row
    bool bad[S];                            // paged: the table named a page outside the pool
    static_for<S>([&](auto si) {
        constexpr int s = decltype(si)::value;
        bad[s] = false;
        send[s] = 0;
        ntl[s] = 0;
        row0[s] = 0;
        tbl[s] = p.block_table;
        if (s < nseg) {
            send[s] = min(sg[s].pos1, sg[s].L - 1);
            ntl[s] = send[s] > sg[s].pos0 ? (send[s] - sg[s].pos0 + 15) >> 4 : 0;
            if constexpr (PG)
                tbl[s] = p.block_table + (size_t)sg[s].b * p.max_pages;
            else
                row0[s] = ((size_t)sg[s].b * p.Hkv + sg[s].j) * p.Lmax;
        }
    });
    const int n0 = ntl[0];
    const int ntot = n0 + ntl[1];

    // K and V rows in the load layout: one wave-wide load is RPI whole rows.
    // DEPTH register sets rotate, so each wave has the loads of DEPTH tiles
    // in flight while it works on one (set indices are compile-time).  The
    // descriptor's inputs are selected by segment (scalar selects, no
    // branch), so that every path issues the same loads in the same order
    // and the compiler's waits before each tile stay partial.  A tile number
    // past the end loads past segment 0's end: nothing is fetched.
    u32x4 kr[DEPTH][VL], vr[DEPTH][VL];
    auto issue = [&](auto set, int i) {
        constexpr int SET = decltype(set)::value;
        const bool valid = i < ntot;
        const bool nxt = valid && i >= n0;
        const int end = nxt ? send[1] : send[0];
        const int base = !valid ? max(send[0], 0) : (nxt ? sg[1].pos0 + 16 * (i - n0) : sg[0].pos0 + 16 * i);
        if constexpr (PG) {
            const int32_t* tb = nxt ? tbl[1] : tbl[0];
            const int jj = nxt ? sg[1].j : sg[0].j;
            bool bf = false;
            const auto kps = page_rsrc(p.k_cache, ROW_BYTES, tb, p, jj, base, end, bf);
            const auto vps = page_rsrc(p.v_cache, ROW_BYTES, tb, p, jj, base, end, bf);
            bad[1] = bad[1] || (nxt && bf);
            bad[0] = bad[0] || (!nxt && bf);
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int off = (u * RPI + r) * ROW_BYTES + c * 16;
                kr[SET][u] = __builtin_amdgcn_raw_buffer_load_b128(kps, off, 0, kStream);
                vr[SET][u] = __builtin_amdgcn_raw_buffer_load_b128(vps, off, 0, kStream);
            }
        } else {
            const size_t row = nxt ? row0[1] : row0[0];
            const uint32_t vb = (uint32_t)max(end, 0) * ROW_BYTES;
            const auto krs = make_rsrc((const char*)p.k_cache + row * ROW_BYTES, vb);
            const auto vrs = make_rsrc((const char*)p.v_cache + row * ROW_BYTES, vb);
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int off = (base + u * RPI + r) * ROW_BYTES + c * 16;
                kr[SET][u] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kStream);
                vr[SET][u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kStream);
            }
        }
    };

    // query operands of S^T, one per segment, shared by the workgroup:
    // column n = head h0 + n (zero past the group), hi and lo halves, in the
    // K tile's layout; one 16-byte piece of one head per thread.  Their
    // loads go out first, so that waiting for them leaves the K/V loads
    // issued next in flight.
    static_assert(16 * LPR <= NTH, "one query piece per thread");
    const int qcol = threadIdx.x / LPR;
    const int qpc = threadIdx.x - qcol * LPR;
    // (without a bias the same offset is read from q, in bounds, and unused:
    // no branch, so nothing waits for these loads before the K/V issue)
    const uint16_t* bsrc = (const uint16_t*)(p.bias ? p.bias : p.q);
    u32x4 qraw[S], braw[S];
    bool qload[S];
    static_for<S>([&](auto si) {
        constexpr int s = decltype(si)::value;
        qraw[s] = u32x4{0u, 0u, 0u, 0u};
        braw[s] = u32x4{0u, 0u, 0u, 0u};
        qload[s] = false;
        if (s < nseg) {
            const int hh = min(HP, p.G - sg[s].hgi * HP);
            qload[s] = threadIdx.x < 16 * LPR && qcol < hh;
            const size_t qh = (size_t)sg[s].j * p.G + sg[s].hgi * HP + min(qcol, hh - 1);
            if (qload[s]) {
                qraw[s] = *(const u32x4*)((const uint16_t*)p.q + ((size_t)sg[s].b * p.H + qh) * D + qpc * 8);
                braw[s] = *(const u32x4*)(bsrc + qh * D + qpc * 8);
            }
        }
    });
    // the appended rows' inputs: wave s takes segment s's when the segment
    // holds its unit's last position; loaded now, so that the row is stored
    // and scored while the first tiles are in flight (without a bias the
    // offsets fall back to valid ones, unused)
    bool new_here = false;
    int nb = 0, nj = 0, nhgi = 0, nL = 1;
    static_for<S>([&](auto si) {
        constexpr int s = decltype(si)::value;
        if (s < nseg && wave == s && sg[s].pos1 == sg[s].L) {
            new_here = true;
            nb = sg[s].b;
            nj = sg[s].j;
            nhgi = sg[s].hgi;
            nL = sg[s].L;
        }
    });
    u32x4 nk = u32x4{0u, 0u, 0u, 0u}, nv = nk, nbk = nk, nbv = nk;
    if (new_here) {
        const size_t src = ((size_t)nb * p.Hkv + nj) * D + c * EPL;
        nk = *(const u32x4*)((const uint16_t*)p.k_new + src);
        nv = *(const u32x4*)((const uint16_t*)p.v_new + src);
        const uint16_t* bb = (const uint16_t*)(p.bias ? p.bias : p.k_new);
        nbk = *(const u32x4*)(bb + (p.bias ? (size_t)(p.H + nj) * D : 0) + c * EPL);
        nbv = *(const u32x4*)(bb + (p.bias ? (size_t)(p.H + p.Hkv + nj) * D : 0) + c * EPL);
    }

    // this wave's share of a round and where it starts; the tile of its
    // k-th turn
    static_assert(NW == 8, "four older and four younger waves");
    const bool older = wave < 4;
    const int share = older ? p.skew_a : p.skew_b;
    const int first = older ? wave * p.skew_a : 4 * p.skew_a + (wave - 4) * p.skew_b;
    const int round = 4 * (p.skew_a + p.skew_b);
    auto tile_of = [&](int k) { return (k / share) * round + first + k % share; };
    // the turn and tile in each register set
    int turn[DEPTH], tidx[DEPTH];
    static_for<DEPTH>([&](auto set) {
        turn[decltype(set)::value] = decltype(set)::value;
        tidx[decltype(set)::value] = tile_of(decltype(set)::value);
        issue(set, tidx[decltype(set)::value]);
    });
    __builtin_amdgcn_sched_barrier(0);

    if (threadIdx.x < 16 * LPR) {
        static_for<S>([&](auto si) {
            constexpr int s = decltype(si)::value;
            if (s < nseg) {
                float x[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
                if (qload[s]) {
                    Elem<KV>::unpack(qraw[s], x);
                    if (p.bias) {
                        float bx[8];
                        Elem<KV>::unpack(braw[s], bx);
#pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] = x[e] + bx[e];
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= p.qscale;
                }
                vec8 hi, lo;
                MF::split8(x, hi, lo);
                unsigned char* qb = qbufs + s * LD::QBYTES;
                *(vec8*)(qb + qcol * LD::KPITCH + qpc * 16) = hi;
                *(vec8*)(qb + 16 * LD::KPITCH + qcol * LD::KPITCH + qpc * 16) = lo;
            }
        });
    }
    __syncthreads();

    // the appended row: stored, and kept as one more softmax state of its
    // segment (score from the staged query halves, as for every other row)
    if (new_here) {
        float kx[EPL], vx[EPL], bx[EPL], ks, vs;
        Elem<KV>::unpack(nk, kx);
        Elem<KV>::unpack(nv, vx);
        if (p.bias) {
            Elem<KV>::unpack(nbk, bx);
#pragma unroll
            for (int e = 0; e < EPL; ++e) kx[e] = kx[e] + bx[e];
            Elem<KV>::unpack(nbv, bx);
#pragma unroll
            for (int e = 0; e < EPL; ++e) vx[e] = vx[e] + bx[e];
        }
        u32x4 kpk, vpk;
        store_new_row<KV, EPL, LPR>(kx, kx, ks, kpk);
        store_new_row<KV, EPL, LPR>(vx, vx, vs, vpk);
        size_t nrow, splane;
        const bool ok = new_row_index<PG>(p, nb, nj, nL - 1, nrow, splane);
        if (ok && nhgi == 0 && r == 0) {
            *(u32x4*)((char*)p.k_cache + nrow * ROW_BYTES + c * 16) = kpk;
            *(u32x4*)((char*)p.v_cache + nrow * ROW_BYTES + c * 16) = vpk;
        }
        const unsigned char* qb = qbufs + wave * LD::QBYTES;
        float* newo = sm_newo + wave * HP * D;
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            float qh[8], ql[8];
            Elem<KV>::unpack(*(const u32x4*)(qb + h * LD::KPITCH + c * 16), qh);
            Elem<KV>::unpack(*(const u32x4*)(qb + 16 * LD::KPITCH + h * LD::KPITCH + c * 16), ql);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(qh[e] + ql[e], kx[e], d);
            d = group_sum<LPR>(d);
            if (r == 0) {
                if (c == 0) {
                    sm_nm[wave][h] = d;
                    sm_nl[wave][h] = ok ? 1.0f : __builtin_nanf("");
                }
#pragma unroll
                for (int e = 0; e < EPL; ++e) newo[h * D + c * EPL + e] = vx[e];
            }
        }
    }

    float m[S], l[S];                       // head n: running max (same in all four quads), this lane's share of the sum
    f32x4 acc[S][DT];                       // O[head 4g+i][16*tn + n]
    static_for<S>([&](auto si) {
        constexpr int s = decltype(si)::value;
        m[s] = kNegInf;
        l[s] = 0.0f;
#pragma unroll
        for (int tn = 0; tn < DT; ++tn) acc[s][tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    });

    // the softmax of one 16-position tile of segment s starting at tb,
    // staged in this wave's LDS tiles
    auto compute = [&](auto si, int tb) {
        constexpr int s = decltype(si)::value;
        const unsigned char* qbuf = qbufs + s * LD::QBYTES;
        // S^T: row = position 4g+i of the tile, column = head n
        f32x4 st = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int piece = (kk * 4 + g) * 16;
            const vec8 ka = MF::bits8(*(const u32x4*)(ktile + n * LD::KPITCH + piece));
            const vec8 qh = MF::bits8(*(const u32x4*)(qbuf + n * LD::KPITCH + piece));
            const vec8 ql = MF::bits8(*(const u32x4*)(qbuf + 16 * LD::KPITCH + n * LD::KPITCH + piece));
            st = MF::mma32(ka, qh, st);
            st = MF::mma32(ka, ql, st);
            // one step's operands live at a time (registers hold the next
            // tiles' loads and the accumulators)
            __builtin_amdgcn_sched_barrier(0);
        }

        // online softmax per head (column n) over the positions of the tile
        float sc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = tb + 4 * g + i < send[s] ? st[i] : kNegInf;
        float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m[s], mt);
        const float ms = mn == kNegInf ? 0.0f : mn;
        const float alpha = fast_exp2(m[s] - ms);
        m[s] = mn;
        float ls = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = fast_exp2(sc[i] - ms);
            ls += sc[i];
        }
        l[s] = l[s] * alpha + ls;
        // P as the A operand of O += P.V: row = head n, k = positions 4g+i
        vec4 ph, pl;
        MF::split4(sc, ph, pl);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
            for (int tn = 0; tn < DT; ++tn) acc[s][tn][i] *= ai;
        }
        // B operand V[position 4g+i][16*tn + n]: one transposing read per
        // 16 columns; lane n of group g names row 4g + n/4, columns 4(n%4)..+3
        const unsigned char* vrow = vtile + (4 * g + (n >> 2)) * LD::VPITCH + (n & 3) * 8;
#pragma unroll
        for (int tn = 0; tn < DT; ++tn) {
            const s16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vrow + tn * 32));
            const vec4 vb = __builtin_bit_cast(vec4, tv);
            acc[s][tn] = MF::mma16(ph, vb, acc[s][tn]);
            acc[s][tn] = MF::mma16(pl, vb, acc[s][tn]);
            if (tn & 1) __builtin_amdgcn_sched_barrier(0);
        }
    };
    // one tile from register set `set`: stage it in LDS, send the loads of
    // this wave's tile DEPTH tiles ahead, then compute (a number past the
    // end only stages and issues: it fetches nothing)
    auto tile = [&](auto set) {
        constexpr int SET = decltype(set)::value;
        lds_wave_fence();
        const int cur = tidx[SET];
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            *(u32x4*)(ktile + (u * RPI + r) * LD::KPITCH + c * 16) = kr[SET][u];
            *(u32x4*)(vtile + (u * RPI + r) * LD::VPITCH + c * 16) = vr[SET][u];
        }
        __builtin_amdgcn_sched_barrier(0);
        turn[SET] += DEPTH;
        const int ni = tile_of(turn[SET]);
        issue(set, ni);
        tidx[SET] = ni;
        __builtin_amdgcn_sched_barrier(0);
        lds_wave_fence();
        if (cur < n0)
            compute(std::integral_constant<int, 0>{}, sg[0].pos0 + 16 * cur);
        else if (cur < ntot)
            compute(std::integral_constant<int, 1>{}, sg[1].pos0 + 16 * (cur - n0));
    };
    // DEPTH tiles per trip with no exit in between, so that the waits the
    // compiler places before each tile's registers stay partial; the trips
    // go on while a set holds a tile of the group
    for (;;) {
        bool any = false;
        static_for<DEPTH>([&](auto set) { any = any || tidx[decltype(set)::value] < ntot; });
        if (!any) break;
        static_for<DEPTH>([&](auto set) { tile(set); });
    }

    // per segment: merge the waves' states and the appended row's; write
    // out, or the piece's partial slot (the workgroup's first segment takes
    // its first slot, any later piece its second).  Every segment's states
    // go to LDS at once, so one barrier serves them all.
    __syncthreads();                        // every wave is done with its tiles
    float* sm_o = (float*)tiles;            // [S][NW][HP][D]
    static_for<S>([&](auto si) {
        constexpr int s = decltype(si)::value;
        if (s < nseg) {
            // l over the four quads of the column
            float ls = l[s];
            ls += __shfl_xor(ls, 16);
            ls += __shfl_xor(ls, 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 4 * g + i;
                if (h < HP) {
#pragma unroll
                    for (int tn = 0; tn < DT; ++tn)
                        sm_o[((s * NW + wave) * HP + h) * D + tn * 16 + n] = acc[s][tn][i];
                }
            }
            if (g == 0 && n < HP) {
                sm_m[s][wave][n] = m[s];
                sm_l[s][wave][n] = bad[s] ? __builtin_nanf("") : ls;   // a page outside the pool: NaN result
            }
        }
    });
    __syncthreads();
    static_for<S>([&](auto si) {
        constexpr int s = decltype(si)::value;
        if (s < nseg) {
            const bool own = sg[s].pos1 == sg[s].L;
            const int h0 = sg[s].j * p.G + sg[s].hgi * HP;
            const int heads_here = min(HP, p.G - sg[s].hgi * HP);
            const int slot = 2 * blk + (first_group && s == 0 ? 0 : 1);
            const float* newo = sm_newo + s * HP * D;
            for (int idx = threadIdx.x; idx < HP * D; idx += NTH) {
                const int h = idx / D;
                const int d = idx - h * D;
                if (h >= heads_here) continue;
                // every wave's state first, as independent reads, so that
                // their latencies overlap instead of adding up
                float mw[NW + 1], lw[NW + 1], ow[NW + 1];
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    mw[w] = sm_m[s][w][h];
                    lw[w] = sm_l[s][w][h];
                    ow[w] = sm_o[((s * NW + w) * HP + h) * D + d];
                }
                // the appended row's state (a weight of zero when the
                // segment does not hold it)
                mw[NW] = own ? sm_nm[s][h] : kNegInf;
                lw[NW] = own ? sm_nl[s][h] : 0.0f;
                ow[NW] = own ? newo[h * D + d] : 0.0f;
                __builtin_amdgcn_sched_barrier(0);
                float M = mw[NW];
#pragma unroll
                for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w]);
                const float ms = M == kNegInf ? 0.0f : M;
                float lsum = 0.0f, o = 0.0f;
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                    const float a = fast_exp2(mw[w] - ms);
                    lsum += a * lw[w];
                    o += a * ow[w];
                }
                if (own) {
                    const float a = fast_exp2(mw[NW] - ms);
                    lsum += a * lw[NW];
                    o += a * ow[NW];
                }
                if (npieces[s] == 1) {
                    A::st(p.out, ((size_t)sg[s].b * p.H + h0 + h) * D + d, o / lsum);
                } else {
                    const size_t sl = (size_t)slot * HP + h;
                    coherent_store(&p.ws_o[sl * D + d], o);
                    if (d == 0) {
                        coherent_store(&p.ws_ml[sl * 2], M);
                        coherent_store(&p.ws_ml[sl * 2 + 1], lsum);
                    }
                }
            }
        }
    });
    __syncthreads();                        // the merge buffers are reused next
}

// Streamed 16-row tiles of a unit of length L: rows [0, L - 1) come from the
// cache, the appended row is handled apart; at least one tile, so that a
// unit of length 1 still has a place in the schedule.
__device__ __forceinline__ int gqa_tiles(int L) { return max(1, (L + 14) >> 4); }

// Grouped-query pass with a range schedule.  The work of a step is the
// 16-row tiles of every unit u = (b, j, hgi) plus `unit_cost` virtual tiles
// per unit that stand for a segment's fixed costs.  Units lie end to end in
// (b, j, hgi) order, and workgroup k takes the tiles [k tpw, (k + 1) tpw),
// tpw = max(ceil(total / grid), range_min), so every workgroup streams about
// the same number of rows whatever the lengths.  A range may cross units:
// the workgroup streams its part of each unit (a segment), up to
// kGqaMaxSeg segments at a time with no barrier between them.  A unit
// inside one range writes `out` directly.  Otherwise each piece writes its
// state to a partial slot (two per workgroup: its first and its last
// segment, the only ones that can be pieces), and the workgroup that
// completes the unit's count merges them.  Partials move between XCDs as
// device-coherent accesses, so no cache-wide writeback or invalidate is
// needed.
template <int KV, int D, int HP, int NW, bool PG>
__global__ void __launch_bounds__(64 * NW) gqa_kernel(const Params p) {
    using A = Act<KV>;
    using LD = GqaLds<D>;
    constexpr int NTH = 64 * NW;
    constexpr int S = kGqaMaxSeg;
    constexpr int O_BYTES = NW * HP * D * 4;
    constexpr int SMEM = cmax(NW * LD::WAVE, O_BYTES);
    static_assert(HP == 4 || HP == 8, "4 or 8 heads per pass");
    static_assert(S <= NW, "one wave per segment handles its appended row");
    static_assert(S * O_BYTES <= SMEM, "every segment's wave states fit in the tile buffers");

    // per-wave tiles while streaming; the merge buffers afterwards
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __shared__ __attribute__((aligned(16))) unsigned char qbufs[S * LD::QBYTES];
    __shared__ float sm_m[S][NW][HP];       // the waves' states, per segment
    __shared__ float sm_l[S][NW][HP];
    __shared__ float sm_nm[S][HP];          // the appended rows' states, per segment
    __shared__ float sm_nl[S][HP];
    __shared__ float sm_newo[S * HP * D];
    __shared__ int sm_last;

    const int lane = threadIdx.x & 63;
    const int upb = p.Hkv * p.n_hg;         // units per sequence
    const int cost = p.unit_cost;
    const int blk = blockIdx.x;
    const int nwg = gridDim.x;

    // Every wave derives the schedule on its own, in registers (no LDS, no
    // barrier): lane l holds sequences l, l + 64, ...; valid lengths, then
    // the total tiles and the range length tpw.
    constexpr int NCH = kGqaMaxBatch / 64;
    int len[NCH];
    int tot = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        len[ch] = 0;
        if (ch * 64 < p.B) {
            const int idx = ch * 64 + lane;
            int Lb = 0;
            if (idx < p.B) {
                Lb = p.seq_lens ? p.seq_lens[idx] : p.step;
                Lb = (Lb >= 1 && Lb <= p.step) ? Lb : 0;
            }
            len[ch] = Lb;
            tot += Lb > 0 ? gqa_tiles(Lb) + cost : 0;
        }
    }
    tot = __builtin_amdgcn_readfirstlane(wave_sum_int(tot)) * upb;
    const int tpw = max((tot + nwg - 1) / nwg, p.range_min);

    // NaN rows for sequences whose length is invalid (no append for them):
    // block bb < B checks sequence bb (the grid has at least B blocks)
    if (blk < p.B) {
        int Lbb = 0;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
            if (ch == blk / 64) Lbb = __builtin_amdgcn_readlane(len[ch], blk % 64);
        if (Lbb == 0)
            for (int idx = threadIdx.x; idx < p.H * D; idx += NTH)
                A::st(p.out, (size_t)blk * p.H * D + idx, __builtin_nanf(""));
    }
    const int t0 = blk * tpw;
    if (t0 >= tot) return;                  // no range for this workgroup
    const int t1 = min(t0 + tpw, tot);

    // the sequence whose units hold tile t0: a scan over the sequences' spans
    int carry = 0, b = -1, pre = 0, L = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        if (ch * 64 < p.B) {
            const int v = len[ch] > 0 ? (gqa_tiles(len[ch]) + cost) * upb : 0;
            int incl = v;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(incl, off);
                if (lane >= off) incl += t;
            }
            const bool hit = t0 >= carry + incl - v && t0 < carry + incl;
            const unsigned long long m = __ballot(hit);
            if (m) {
                const int l = __builtin_ctzll(m);
                b = ch * 64 + l;
                pre = carry + __builtin_amdgcn_readlane(incl - v, l);
                L = __builtin_amdgcn_readlane(len[ch], l);
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
    }
    // the schedule, the same in every wave: scalar registers, so that the
    // loop bounds, the descriptors and block-table reads stay scalar
    b = __builtin_amdgcn_readfirstlane(b);
    if (b < 0) return;
    L = __builtin_amdgcn_readfirstlane(L);
    pre = __builtin_amdgcn_readfirstlane(pre);
    int nt = gqa_tiles(L);
    int ub = (t0 - pre) / (nt + cost);      // unit within the sequence: j * n_hg + hgi
    int vu = pre + ub * (nt + cost);        // the unit's first (virtual) tile
    bool done = false;

    // the pieces among this workgroup's segments: unit, its first virtual
    // tile, its first piece's workgroup, its number of pieces
    int np = 0;
    int pu0 = 0, pv0 = 0, pk0 = 0, pn0 = 0, pu1 = 0, pv1 = 0, pk1 = 0, pn1 = 0;
    for (bool first_group = true;; first_group = false) {
        // the next (up to) kGqaMaxSeg segments of the range
        GqaSeg sg[S];
        int npc[S];
        int nseg = 0;
        static_for<S>([&](auto si) {
            constexpr int s = decltype(si)::value;
            sg[s] = GqaSeg{0, 0, 0, 1, 0, 0};
            npc[s] = 1;
            if (!done) {
                const int rs = vu + cost;   // the unit's streamed tiles [rs, re)
                const int re = rs + nt;
                if (rs >= t1) {
                    done = true;
                } else {
                    const int s0 = max(rs, t0), s1 = min(re, t1);
                    const int j = ub / p.n_hg;
                    sg[s] = GqaSeg{b, j, ub - j * p.n_hg, L, (s0 - rs) * 16, s1 == re ? L : (s1 - rs) * 16};
                    const int kf = rs / tpw;
                    npc[s] = (re - 1) / tpw - kf + 1;
                    if (npc[s] > 1) {
                        if (np == 0) {
                            pu0 = b * upb + ub; pv0 = vu; pk0 = kf; pn0 = npc[s];
                        } else {
                            pu1 = b * upb + ub; pv1 = vu; pk1 = kf; pn1 = npc[s];
                        }
                        ++np;
                    }
                    nseg = s + 1;
                    // the next unit: the next head group or KV head, else
                    // the next valid sequence
                    vu = re;
                    if (++ub == upb) {
                        ub = 0;
                        int nb = -1, nl = 0;
#pragma unroll
                        for (int ch = 0; ch < NCH; ++ch) {
                            if (ch * 64 < p.B && nb < 0) {
                                const unsigned long long m = __ballot(ch * 64 + lane > b && len[ch] > 0);
                                if (m) {
                                    const int l = __builtin_ctzll(m);
                                    nb = ch * 64 + l;
                                    nl = __builtin_amdgcn_readlane(len[ch], l);
                                }
                            }
                        }
                        if (nb < 0) {
                            done = true;
                        } else {
                            b = __builtin_amdgcn_readfirstlane(nb);
                            L = __builtin_amdgcn_readfirstlane(nl);
                            nt = gqa_tiles(L);
                        }
                    }
                }
            }
        });
        if (nseg == 0) break;
        gqa_group<KV, D, HP, NW, PG>(p, smem, qbufs, sm_m, sm_l, sm_nm, sm_nl, sm_newo, sg, npc, nseg, blk,
                                     first_group);
        if (done) break;
    }
    if (np == 0) return;

    // partials are written through to the device coherence point; once every
    // thread's stores are acknowledged the units' counts go up, and the
    // workgroup that completes a count reads the unit's partials back
    // coherently and merges them.
    // Ordering: the partials are agent-scope atomic stores and loads, which
    // gfx950 performs at the device coherence point (past the per-XCD L2),
    // so no cache holds a stale or dirty copy of them.  A store counts as
    // done (vmcnt) only once that point has acknowledged it, so after
    // wait_stores and the barrier every partial of this workgroup is
    // visible device-wide before thread 0's count increment is issued; the
    // reader issues its loads only after its own increment has returned the
    // completed count.  A release/acquire increment would add an L2
    // writeback and invalidate (buffer_wbl2, buffer_inv) that these
    // write-through accesses do not need; it measured 61.5 against 57.5 us
    // on the ragged grouped-query workload.
    wait_stores();
    __syncthreads();
    for (int i = 0; i < np; ++i) {
        const int unit = i == 0 ? pu0 : pu1;
        const int uv = i == 0 ? pv0 : pv1;
        const int kf = i == 0 ? pk0 : pk1;
        const int npieces = i == 0 ? pn0 : pn1;
        if (threadIdx.x == 0)
            sm_last = __hip_atomic_fetch_add(&p.counters[unit], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == npieces - 1;
        __syncthreads();
        const bool last = sm_last;
        __syncthreads();                    // sm_last is written again for the next unit
        if (!last) continue;
        const int ub2 = unit % upb;
        const int b2 = unit / upb;
        const int j = ub2 / p.n_hg;
        const int hgi = ub2 - j * p.n_hg;
        const int h0 = j * p.G + hgi * HP;
        const int heads_here = min(HP, p.G - hgi * HP);
        // piece k of the unit sits in workgroup kf + k, in that workgroup's
        // first slot, except the first piece when the workgroup's range
        // began in an earlier unit (then it is the workgroup's last segment)
        const int slot_first = 2 * kf + (uv > kf * tpw ? 1 : 0);
        // each output reads every piece's (m, l, o) with independent loads,
        // four pieces per round, and merges them with a running maximum
        for (int idx = threadIdx.x; idx < HP * D; idx += NTH) {
            const int h = idx / D;
            const int d = idx - h * D;
            if (h >= heads_here) continue;
            float M = kNegInf, lsum = 0.0f, o = 0.0f;
            for (int k0 = 0; k0 < npieces; k0 += 4) {
                float mk[4], lk[4], ok[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int k = min(k0 + q, npieces - 1);
                    const size_t sl = (size_t)(k == 0 ? slot_first : 2 * (kf + k)) * HP + h;
                    mk[q] = coherent_load(&p.ws_ml[sl * 2]);
                    lk[q] = coherent_load(&p.ws_ml[sl * 2 + 1]);
                    ok[q] = coherent_load(&p.ws_o[sl * D + d]);
                }
                float Mn = M;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < npieces) Mn = fmaxf(Mn, mk[q]);
                const float ms = Mn == kNegInf ? 0.0f : Mn;
                const float a = fast_exp2(M - ms);
                lsum *= a;
                o *= a;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (k0 + q < npieces) {
                        const float w = fast_exp2(mk[q] - ms);
                        lsum += w * lk[q];
                        o += w * ok[q];
                    }
                }
                M = Mn;
            }
            A::st(p.out, ((size_t)b2 * p.H + h0 + h) * D + d, o / lsum);
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(&p.counters[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();                    // LDS is reused by the next unit's merge
    }
}

// ---------------------------------------------------------------------------
// Combine: one wave per (b, h).  out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// ---------------------------------------------------------------------------
template <int KV, int D>
__global__ void __launch_bounds__(kThreads) combine_kernel(const Params p) {
    using A = Act<KV>;
    constexpr int EL = D / 64;
    const int lane = threadIdx.x & 63;
    const int bh = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (bh >= p.B * p.H) return;
    const int b = bh / p.H;
    const int L = __builtin_amdgcn_readfirstlane(p.seq_lens ? p.seq_lens[b] : p.step);
    if (L < 1 || L > p.step) {
#pragma unroll
        for (int e = 0; e < EL; ++e) A::st(p.out, (size_t)bh * D + lane * EL + e, __builtin_nanf(""));
        return;
    }
    const int n_chunks = (L + p.chunk - 1) / p.chunk;
    const float* ml = p.ws_ml + (size_t)bh * p.S * 2;
    const float* wo = p.ws_o + (size_t)bh * p.S * D;
    float M = kNegInf;
    for (int s = lane; s < n_chunks; s += 64) M = fmaxf(M, ml[2 * s]);
    M = wave_max(M);
    float lsum = 0.0f;
    for (int s = lane; s < n_chunks; s += 64) lsum += fast_exp2(ml[2 * s] - M) * ml[2 * s + 1];
    lsum = wave_sum(lsum);
    float acc[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] = 0.0f;
#pragma unroll 4
    for (int s = 0; s < n_chunks; ++s) {
        const float a = fast_exp2(ml[2 * s] - M);
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[e] = fmaf(a, wo[(size_t)s * D + lane * EL + e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) A::st(p.out, (size_t)bh * D + lane * EL + e, acc[e] / lsum);
}

constexpr int unroll_for(int gt) { return gt <= 2 ? 8 : 4; }
// 16-wave workgroups cap a wave at 128 registers; only the one-head passes
// of the fp32/fp16/bf16 caches fit without spilling.
constexpr bool wide_built(int kv, int gt) { return gt == 1 && kv != KV_I8; }

constexpr int kGqaWaves = 8;
constexpr int kGqaBlocksPerCu = 1;   // ranges per CU (one 8-wave workgroup: about 98 KiB of LDS at D = 128)
// Virtual tiles charged per unit for a segment's fixed costs (a tile is 16
// rows, about 0.3 us of one CU's share of the bandwidth); 16 measured best
// over 0..32 on ragged lengths.
constexpr int kGqaUnitCost = 16;
// Tiles per round for each older and each younger wave: a SIMD serves its
// older wave first, and a younger wave left alone at the end streams more
// slowly; 2:1 and 3:2 measured best of 1:1, 2:1, 3:2, 4:3 and 8:7 on ragged
// lengths, 2:1 by a little with the charge of 16.
constexpr int kGqaSkewA = 2;
constexpr int kGqaSkewB = 1;

template <int KV, int D, int HP, bool PG>
hipError_t launch_gqa_t(const Params& p, hipStream_t s) {
    hipLaunchKernelGGL((gqa_kernel<KV, D, HP, kGqaWaves, PG>), dim3(p.S), dim3(64 * kGqaWaves), 0, s, p);
    return hipGetLastError();
}

template <int KV, int D, int GT, bool PG, bool LP>
hipError_t launch_attention_lp(const Params& p, int nw, hipStream_t s) {
    dim3 grid(p.S, p.Hkv * p.n_hg, p.B);
    constexpr int U = unroll_for(GT);
    if constexpr (wide_built(KV, GT)) {
        if (nw == 16) {
            hipLaunchKernelGGL((attention_kernel<KV, D, GT, U, 16, PG, LP>), grid, dim3(64 * 16), 0, s, p);
            return hipGetLastError();
        }
    }
    if (nw != 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attention_kernel<KV, D, GT, U, 4, PG, LP>), grid, dim3(64 * 4), 0, s, p);
    return hipGetLastError();
}

template <int KV, int D, int GT, bool PG>
hipError_t launch_attention_t(const Params& p, int nw, hipStream_t s) {
    if constexpr ((KV == KV_F16 || KV == KV_BF16) && (GT == 4 || GT == 8)) {
        if (p.balanced) return launch_gqa_t<KV, D, GT, PG>(p, s);
    }
    if constexpr (PG) {
        // rows one wave loads per iteration (the same for both workgroup shapes)
        constexpr int ELEM = KV == KV_F32 ? 4 : (KV == KV_I8 ? 1 : 2);
        constexpr int WAVE_ROWS = 64 / (D * ELEM / 16) * unroll_for(GT);
        if ((1 << p.page_shift) >= WAVE_ROWS) return launch_attention_lp<KV, D, GT, true, true>(p, nw, s);
        return launch_attention_lp<KV, D, GT, true, false>(p, nw, s);
    } else {
        return launch_attention_lp<KV, D, GT, false, false>(p, nw, s);
    }
}

template <int KV, int D, bool PG>
hipError_t dispatch_gt(const Params& p, int gt, int nw, hipStream_t s) {
    switch (gt) {
    case 1: return launch_attention_t<KV, D, 1, PG>(p, nw, s);
    case 2: return launch_attention_t<KV, D, 2, PG>(p, nw, s);
    case 4: return launch_attention_t<KV, D, 4, PG>(p, nw, s);
    case 8: return launch_attention_t<KV, D, 8, PG>(p, nw, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KV>
hipError_t dispatch_d(const Params& p, int d, int gt, int nw, hipStream_t s) {
    const bool pg = p.block_table != nullptr;
    switch (d) {
    case 64: return pg ? dispatch_gt<KV, 64, true>(p, gt, nw, s) : dispatch_gt<KV, 64, false>(p, gt, nw, s);
    case 128: return pg ? dispatch_gt<KV, 128, true>(p, gt, nw, s) : dispatch_gt<KV, 128, false>(p, gt, nw, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KV, int D>
hipError_t launch_combine_t(const Params& p, hipStream_t s) {
    const int blocks = (p.B * p.H + kWaves - 1) / kWaves;
    hipLaunchKernelGGL((combine_kernel<KV, D>), dim3(blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int group_tile(int G) {
    if (G >= 8) return 8;
    int t = 1;
    while (t < G) t <<= 1;
    return t;
}

int gqa_blocks_per_cu() {
    const int v = tuning().gqa_blocks_per_cu;
    return v > 0 && v <= 16 ? v : kGqaBlocksPerCu;
}

void gqa_skew(int& a, int& b) {
    const Tuning& t = tuning();
    const bool set = t.gqa_skew_a >= 1 && t.gqa_skew_a <= 16 && t.gqa_skew_b >= 1 && t.gqa_skew_b <= 16;
    a = set ? t.gqa_skew_a : kGqaSkewA;
    b = set ? t.gqa_skew_b : kGqaSkewB;
}

int gqa_unit_cost() {
    const int v = tuning().gqa_unit_cost;
    return v >= 0 && v <= 64 ? v : kGqaUnitCost;
}

bool use_gqa_mfma(int kv, int gtile, int batch) {
    if (!((kv == KV_F16 || kv == KV_BF16) && (gtile == 4 || gtile == 8))) return false;
    if (batch > kGqaMaxBatch) return false;
    return tuning().gqa_valu != 1;
}

int tile_rows(int kv, int head_dim, int gtile, int nw) {
    const int bytes = kv == KV_F32 ? 4 : (kv == KV_I8 ? 1 : 2);
    const int lpr = head_dim * bytes / 16;
    return nw * (64 / lpr) * unroll_for(gtile);
}

bool wide_ok(int kv, int gtile) { return wide_built(kv, gtile); }

hipError_t launch_attention(const Params& p, int kv, int head_dim, int gtile, int nw, hipStream_t s) {
    switch (kv) {
    case KV_F32: return dispatch_d<KV_F32>(p, head_dim, gtile, nw, s);
    case KV_F16: return dispatch_d<KV_F16>(p, head_dim, gtile, nw, s);
    case KV_BF16: return dispatch_d<KV_BF16>(p, head_dim, gtile, nw, s);
    case KV_I8: return dispatch_d<KV_I8>(p, head_dim, gtile, nw, s);
    default: return hipErrorInvalidValue;
    }
}

namespace {
__global__ void __launch_bounds__(256) zero_ints_kernel(int* dst, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = 0;
}
}  // namespace

hipError_t launch_zero_ints(int* dst, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, n);
    return hipGetLastError();
}

hipError_t static_scratch(int device, hipStream_t s, void** ptr) {
    static std::mutex m;
    static std::map<int, void*> addr;      // device -> its copy of `scratch`
    std::lock_guard<std::mutex> lock(m);
    auto it = addr.find(device);
    if (it != addr.end()) {
        *ptr = it->second;
        return hipSuccess;
    }
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // the counters must start at zero; every call of the grouped-query pass
    // leaves them at zero again
    e = launch_zero_ints((int*)p, kStaticCounterInts, s);
    if (e != hipSuccess) return e;
    addr[device] = p;
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_combine(const Params& p, int kv, int head_dim, hipStream_t s) {
#define FTM_COMBINE_CASE(K)                                               \
    case K:                                                               \
        return head_dim == 64 ? launch_combine_t<K, 64>(p, s)             \
                              : launch_combine_t<K, 128>(p, s);
    switch (kv) {
        FTM_COMBINE_CASE(KV_F32)
        FTM_COMBINE_CASE(KV_F16)
        FTM_COMBINE_CASE(KV_BF16)
        FTM_COMBINE_CASE(KV_I8)
    default: return hipErrorInvalidValue;
    }
#undef FTM_COMBINE_CASE
}

}  // namespace ftm
