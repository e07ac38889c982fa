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
#include <cstdlib>

#include "gfx950.hpp"

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

// ---------------------------------------------------------------------------
// Cross-lane reductions.  A cache row is held by LPR consecutive lanes
// (LPR in {4, 8, 16, 32}); the all-reduce over those lanes stays inside a
// DPP row where it can: quad swaps, then the half-row mirror (8 lanes) or
// rotations by 4 and 8 (16 lanes); a 32-lane row adds one cross-row swap.
// ---------------------------------------------------------------------------
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

template <int LPR> __device__ __forceinline__ float group_sum(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    if constexpr (LPR == 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (LPR >= 16) {
        v += dpp<kRowRor4>(v);
        v += dpp<kRowRor8>(v);
    }
    if constexpr (LPR == 32) v += __shfl_xor(v, 16);
    return v;
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
template <int KV, int D, int GT, int U, int NW, bool PG>
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
    // powers of two, base a multiple of RPI)
    auto issue_stream = [&](const void* pool, const __amdgpu_buffer_rsrc_t& rs,
                            const __amdgpu_buffer_rsrc_t& srs, size_t splane, u32x4* dst,
                            float* sdst, int base) {
        if constexpr (PG) {
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

// Largest batch the balanced schedule handles (its per-sequence work
// offsets live in LDS); larger batches take the vector-ALU pass.
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

// One segment [pos0, pos1) of one unit (sequence b, KV head j, head group
// hgi) streamed by the whole workgroup.  On return the workgroup's states
// sit in LDS: n_states softmax states (m, l, o[HP][D]), one per wave (o in
// `tiles`) plus, when the segment holds the new row, the appended row's
// (m and l in slot NW, o in sm_newo).
template <int KV, int D, int HP, int NW, bool PG>
__device__ __forceinline__ int gqa_segment(const Params& p, unsigned char* tiles, unsigned char* qbuf,
                                           float (*sm_m)[HP], float (*sm_l)[HP], float* sm_newo,
                                           int b, int j, int hgi, int L, int pos0, int pos1) {
    using MF = Mfma<KV>;
    using LD = GqaLds<D>;
    typedef typename MF::vec8 vec8;
    typedef typename MF::vec4 vec4;
    constexpr int NTH = 64 * NW;
    constexpr int ROW_BYTES = D * 2;
    constexpr int KK = D / 32;              // S^T: MFMA steps over the head dim
    constexpr int DT = D / 16;              // O: 16-column tiles
    constexpr int EPL = 8;                  // loads: elements per lane
    constexpr int LPR = D / EPL;            // loads: lanes per row
    constexpr int RPI = 64 / LPR;           // loads: rows per wave-wide load
    constexpr int VL = 16 / RPI;            // loads per 16-position tile, each of K and V
    constexpr int BLOCK_ROWS = NW * 16;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;                // MFMA layout: k-slot group, position quad
    const int n = lane & 15;                // MFMA layout: K row / head column / V column
    const int r = lane / LPR;               // load layout: row slot
    const int c = lane % LPR;               // load layout: 16-byte column slice
    const int h0 = j * p.G + hgi * HP;
    const int heads_here = min(HP, p.G - hgi * HP);
    const int stream_end = min(pos1, L - 1);
    const bool owns_new = pos1 == L;

    // contiguous cache: one descriptor per stream over rows [0, stream_end)
    // of this (b, j); paged: one per 16-position tile (tiles start at
    // multiples of 16 and never straddle a page, P >= 16)
    const size_t row0 = ((size_t)b * p.Hkv + j) * p.Lmax;
    const uint32_t valid_bytes = PG ? 0u : (uint32_t)max(stream_end, 0) * ROW_BYTES;
    const auto krs = make_rsrc(PG ? nullptr : (const char*)p.k_cache + row0 * ROW_BYTES, valid_bytes);
    const auto vrs = make_rsrc(PG ? nullptr : (const char*)p.v_cache + row0 * ROW_BYTES, valid_bytes);
    const int32_t* tbl = PG ? p.block_table + (size_t)b * p.max_pages : nullptr;
    bool bad = false;                       // paged: the table named a page outside the pool
    unsigned char* ktile = tiles + wave * LD::WAVE;
    unsigned char* vtile = ktile + 16 * LD::KPITCH;

    // K and V rows in the load layout: one wave-wide load is RPI whole rows.
    // DEPTH register sets rotate, so each wave has the loads of DEPTH tiles
    // in flight while it works on one (set indices are compile-time).
    constexpr int DEPTH = kGqaDepth;
    u32x4 kr[DEPTH][VL], vr[DEPTH][VL];
    auto issue = [&](auto set, int base) {
        constexpr int S = decltype(set)::value;
        if constexpr (PG) {
            const auto kps = page_rsrc(p.k_cache, ROW_BYTES, tbl, p, j, base, stream_end, bad);
            const auto vps = page_rsrc(p.v_cache, ROW_BYTES, tbl, p, j, base, stream_end, bad);
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int off = (u * RPI + r) * ROW_BYTES + c * 16;
                kr[S][u] = __builtin_amdgcn_raw_buffer_load_b128(kps, off, 0, kStream);
                vr[S][u] = __builtin_amdgcn_raw_buffer_load_b128(vps, off, 0, kStream);
            }
        } else {
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int off = (base + u * RPI + r) * ROW_BYTES + c * 16;
                kr[S][u] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kStream);
                vr[S][u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kStream);
            }
        }
    };
    // query operand of S^T, shared by the workgroup: column n = head h0 + n
    // (zero past the group), hi and lo halves, in the K tile's layout; one
    // 16-byte piece of one head per thread.  Its loads go out first, so that
    // waiting for them leaves the K/V loads issued next in flight.
    static_assert(16 * LPR <= NTH, "one query piece per thread");
    const int qcol = threadIdx.x / LPR;
    const int qpc = threadIdx.x - qcol * LPR;
    const bool qload = threadIdx.x < 16 * LPR && qcol < heads_here;
    const size_t qh_idx = (size_t)h0 + min(qcol, heads_here - 1);
    // (without a bias the same offset is read from q, in bounds, and unused:
    // no branch, so nothing waits for these loads before the K/V issue)
    const uint16_t* bsrc = (const uint16_t*)(p.bias ? p.bias : p.q);
    u32x4 qraw = u32x4{0u, 0u, 0u, 0u}, braw = u32x4{0u, 0u, 0u, 0u};
    if (qload) {
        qraw = *(const u32x4*)((const uint16_t*)p.q + ((size_t)b * p.H + qh_idx) * D + qpc * 8);
        braw = *(const u32x4*)(bsrc + qh_idx * D + qpc * 8);
    }
    // the appended row's inputs (the piece holding position L-1, wave 0):
    // loaded now, so the row is stored and scored while the first tiles are
    // in flight (without a bias the offsets fall back to valid ones, unused)
    const bool new_here = owns_new && wave == 0;
    u32x4 nk = u32x4{0u, 0u, 0u, 0u}, nv = nk, nbk = nk, nbv = nk;
    if (new_here) {
        const size_t src = ((size_t)b * p.Hkv + j) * D + c * EPL;
        nk = *(const u32x4*)((const uint16_t*)p.k_new + src);
        nv = *(const u32x4*)((const uint16_t*)p.v_new + src);
        const uint16_t* bb = (const uint16_t*)(p.bias ? p.bias : p.k_new);
        nbk = *(const u32x4*)(bb + (p.bias ? (size_t)(p.H + j) * D : 0) + c * EPL);
        nbv = *(const u32x4*)(bb + (p.bias ? (size_t)(p.H + p.Hkv + j) * D : 0) + c * EPL);
    }

    int base = pos0 + wave * 16;
    static_for<DEPTH>([&](auto set) { issue(set, base + decltype(set)::value * BLOCK_ROWS); });
    __builtin_amdgcn_sched_barrier(0);

    if (threadIdx.x < 16 * LPR) {
        float x[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
        if (qload) {
            Elem<KV>::unpack(qraw, x);
            if (p.bias) {
                float bx[8];
                Elem<KV>::unpack(braw, bx);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = x[e] + bx[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= p.qscale;
        }
        vec8 hi, lo;
        MF::split8(x, hi, lo);
        *(vec8*)(qbuf + qcol * LD::KPITCH + qpc * 16) = hi;
        *(vec8*)(qbuf + 16 * LD::KPITCH + qcol * LD::KPITCH + qpc * 16) = lo;
    }
    __syncthreads();

    // the appended row: stored, and kept as one more softmax state (score
    // from the staged query halves, as for every other row of the pass)
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
        const bool ok = new_row_index<PG>(p, b, j, L - 1, nrow, splane);
        if (ok && hgi == 0 && r == 0) {
            *(u32x4*)((char*)p.k_cache + nrow * ROW_BYTES + c * 16) = kpk;
            *(u32x4*)((char*)p.v_cache + nrow * ROW_BYTES + c * 16) = vpk;
        }
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            float qh[8], ql[8];
            Elem<KV>::unpack(*(const u32x4*)(qbuf + h * LD::KPITCH + c * 16), qh);
            Elem<KV>::unpack(*(const u32x4*)(qbuf + 16 * LD::KPITCH + h * LD::KPITCH + c * 16), ql);
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = fmaf(qh[e] + ql[e], kx[e], d);
            d = group_sum<LPR>(d);
            if (r == 0) {
                if (c == 0) {
                    sm_m[NW][h] = d;
                    sm_l[NW][h] = ok ? 1.0f : __builtin_nanf("");
                }
#pragma unroll
                for (int e = 0; e < EPL; ++e) sm_newo[h * D + c * EPL + e] = vx[e];
            }
        }
    }

    float m = kNegInf;                      // head n: running max (same in all four quads)
    float l = 0.0f;                         // head n: this lane's share of the sum
    f32x4 acc[DT];                          // O[head 4g+i][16*tn + n]
#pragma unroll
    for (int tn = 0; tn < DT; ++tn) acc[tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // one 16-position tile starting at tb, from register set `set`
    auto tile = [&](auto set, int tb) {
        constexpr int S = decltype(set)::value;
        // stage the tile in LDS, then send the loads DEPTH tiles ahead out
        lds_wave_fence();
#pragma unroll
        for (int u = 0; u < VL; ++u) {
            *(u32x4*)(ktile + (u * RPI + r) * LD::KPITCH + c * 16) = kr[S][u];
            *(u32x4*)(vtile + (u * RPI + r) * LD::VPITCH + c * 16) = vr[S][u];
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(set, tb + DEPTH * BLOCK_ROWS);
        __builtin_amdgcn_sched_barrier(0);
        lds_wave_fence();

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
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = tb + 4 * g + i < stream_end ? st[i] : kNegInf;
        float mt = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mt = fmaxf(mt, __shfl_xor(mt, 16));
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mn = fmaxf(m, mt);
        const float ms = mn == kNegInf ? 0.0f : mn;
        const float alpha = fast_exp2(m - ms);
        m = mn;
        float ls = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = fast_exp2(s[i] - ms);
            ls += s[i];
        }
        l = l * alpha + ls;
        // P as the A operand of O += P.V: row = head n, k = positions 4g+i
        vec4 ph, pl;
        MF::split4(s, ph, pl);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
            for (int tn = 0; tn < DT; ++tn) acc[tn][i] *= ai;
        }
        // B operand V[position 4g+i][16*tn + n]: one transposing read per
        // 16 columns; lane n of group g names row 4g + n/4, columns 4(n%4)..+3
        const unsigned char* vrow = vtile + (4 * g + (n >> 2)) * LD::VPITCH + (n & 3) * 8;
#pragma unroll
        for (int tn = 0; tn < DT; ++tn) {
            const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(vrow + tn * 32));
            const vec4 vb = __builtin_bit_cast(vec4, t);
            acc[tn] = MF::mma16(ph, vb, acc[tn]);
            acc[tn] = MF::mma16(pl, vb, acc[tn]);
            if (tn & 1) __builtin_amdgcn_sched_barrier(0);
        }
    };
    // DEPTH tiles per trip with no exit in between, so that the waits the
    // compiler places before each tile's registers stay partial (a tile
    // past the end is all masked: its loads fetch nothing, its weights are 0)
    for (; base < stream_end; base += DEPTH * BLOCK_ROWS)
        static_for<DEPTH>([&](auto set) { tile(set, base + decltype(set)::value * BLOCK_ROWS); });

    // l over the four quads of the column
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    __syncthreads();                        // every wave is done with its tiles
    float* sm_o = (float*)tiles;            // [NW][HP][D]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        if (h < HP) {
#pragma unroll
            for (int tn = 0; tn < DT; ++tn) sm_o[(wave * HP + h) * D + tn * 16 + n] = acc[tn][i];
        }
    }
    if (g == 0 && n < HP) {
        sm_m[wave][n] = m;
        sm_l[wave][n] = bad ? __builtin_nanf("") : l;   // a page outside the pool: NaN result
    }

    __syncthreads();
    return owns_new ? NW + 1 : NW;
}

// Grouped-query pass with a balanced schedule.  The work of a step is L_b
// positions for each unit u = (b, j, hgi).  With W = max(seg_min,
// ceil(total / target)) the units of sequence b are cut into
// n_b = max(1, round(L_b / W)) near-equal pieces, one workgroup per piece,
// so every workgroup streams about W rows whatever the lengths, and each
// streams a single piece (one prologue, one epilogue).  The grid has
// target + units workgroups, at least the number of pieces; the rest exit.
// A unit in one piece writes `out` directly.  Otherwise each piece writes
// its state to the unit's partial slot, and the last piece to finish (an
// atomic count per unit) merges the slots into `out` and clears the count
// for the next call.  Partials move between XCDs as device-coherent
// accesses, so no cache-wide writeback or invalidate is needed.
template <int KV, int D, int HP, int NW, bool PG>
__global__ void __launch_bounds__(64 * NW) gqa_kernel(const Params p) {
    using A = Act<KV>;
    using LD = GqaLds<D>;
    constexpr int NTH = 64 * NW;
    constexpr int O_BYTES = NW * HP * D * 4;
    static_assert(HP == 4 || HP == 8, "4 or 8 heads per pass");

    // per-wave tiles while streaming; the merge buffers afterwards
    __shared__ __attribute__((aligned(16))) unsigned char smem[cmax(NW * LD::WAVE, O_BYTES)];
    __shared__ __attribute__((aligned(16))) unsigned char qbuf[LD::QBYTES];
    __shared__ float sm_m[NW + 1][HP];      // slot NW: the appended row
    __shared__ float sm_l[NW + 1][HP];
    __shared__ float sm_newo[HP * D];       // the appended row's values
    __shared__ int sm_last;

    const int lane = threadIdx.x & 63;
    const int upb = p.Hkv * p.n_hg;         // units per sequence
    const int target = gridDim.x - p.B * upb;

    // Every wave derives the schedule on its own, in registers (no LDS, no
    // barrier): lane l holds sequences l, l + 64, ...; valid lengths, total
    // work, slice length W, pieces per sequence n_b * upb and their prefix,
    // then the sequence whose pieces include this workgroup's.
    constexpr int NCH = kGqaMaxBatch / 64;
    int len[NCH];
    int tot = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int idx = ch * 64 + lane;
        int Lb = 0;
        if (idx < p.B) {
            Lb = p.seq_lens ? p.seq_lens[idx] : p.step;
            Lb = (Lb >= 1 && Lb <= p.step) ? Lb : 0;
        }
        len[ch] = Lb;
        tot += Lb;
    }
    tot = __builtin_amdgcn_readfirstlane(wave_sum_int(tot));
    const long long total = (long long)tot * upb;
    const int W = max((int)((total + target - 1) / max(target, 1)), p.seg_min);
    const int blk = blockIdx.x;
    int carry = 0, b = -1, first = 0, npc = 0, L = 0;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const int v = len[ch] > 0 ? max(1, (len[ch] + W / 2) / W) * upb : 0;
        int incl = v;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const bool hit = blk >= carry + incl - v && blk < carry + incl;
        const unsigned long long m = __ballot(hit);
        if (m) {
            const int l = __builtin_ctzll(m);
            b = ch * 64 + l;
            first = carry + __builtin_amdgcn_readlane(incl - v, l);
            npc = __builtin_amdgcn_readlane(v, l);
            L = __builtin_amdgcn_readlane(len[ch], l);
        }
        carry += __builtin_amdgcn_readlane(incl, 63);
    }

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
    if (b < 0) return;                      // no piece for this workgroup

    // the piece, the same in every wave: scalar registers, so that the loop
    // bounds, the descriptors and block-table reads stay scalar
    b = __builtin_amdgcn_readfirstlane(b);
    L = __builtin_amdgcn_readfirstlane(L);
    const int nseg = __builtin_amdgcn_readfirstlane(npc / upb);
    const int local = __builtin_amdgcn_readfirstlane(blk - first);
    const int ub = local / nseg;            // unit within the sequence: j * n_hg + hgi
    const int seg = local - ub * nseg;
    // piece boundaries on multiples of 16 (a tile never straddles a page)
    const int pos0 = __builtin_amdgcn_readfirstlane(seg == 0 ? 0 : (int)((long long)seg * L / nseg) & ~15);
    const int pos1 = __builtin_amdgcn_readfirstlane(seg == nseg - 1 ? L
                                                    : (int)((long long)(seg + 1) * L / nseg) & ~15);
    const int j = ub / p.n_hg;
    const int hgi = ub - j * p.n_hg;
    const int h0 = j * p.G + hgi * HP;
    const int heads_here = min(HP, p.G - hgi * HP);
    const int unit = b * upb + ub;

    const int n_states = gqa_segment<KV, D, HP, NW, PG>(p, smem, qbuf, sm_m, sm_l, sm_newo, b, j, hgi,
                                                        L, pos0, pos1);
    float* sm_o = (float*)smem;

    // merge this workgroup's states; write out, or the unit's partial slot
    for (int idx = threadIdx.x; idx < HP * D; idx += NTH) {
        const int h = idx / D;
        const int d = idx - h * D;
        if (h >= heads_here) continue;
        float M = sm_m[0][h];
        for (int w = 1; w < n_states; ++w) M = fmaxf(M, sm_m[w][h]);
        const float ms = M == kNegInf ? 0.0f : M;
        float lsum = 0.0f, o = 0.0f;
        for (int w = 0; w < n_states; ++w) {
            const float a = fast_exp2(sm_m[w][h] - ms);
            lsum += a * sm_l[w][h];
            o += a * (w < NW ? sm_o[(w * HP + h) * D + d] : sm_newo[h * D + d]);
        }
        if (nseg == 1) {
            A::st(p.out, ((size_t)b * p.H + h0 + h) * D + d, o / lsum);
        } else {
            const size_t slot = ((size_t)unit * p.seg_max + seg) * HP + h;
            coherent_store(&p.ws_o[slot * D + d], o);
            if (d == 0) {
                coherent_store(&p.ws_ml[slot * 2], M);
                coherent_store(&p.ws_ml[slot * 2 + 1], lsum);
            }
        }
    }
    if (nseg == 1) return;
    // partials are written through to the device coherence point; once every
    // thread's stores are acknowledged the unit's count goes up, and the
    // workgroup that completes it reads the partials back coherently
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        sm_last = __hip_atomic_fetch_add(&p.counters[unit], 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == nseg - 1;
    __syncthreads();
    if (!sm_last) return;
    // one parallel round for the pieces' (m, l), kept in LDS as rescale
    // factors; then each output sums its pieces with independent loads
    const size_t slot0 = (size_t)unit * p.seg_max * HP;
    float* sm_a = (float*)smem;             // [seg_max][HP]: l_k, then the weights 2^(m_k - M)
    float* sm_ls = sm_a + p.seg_max * HP;   // [HP]: 1 / sum_k 2^(m_k - M) l_k
    float* sm_ms = sm_ls + HP;              // [seg_max][HP]: m_k
    for (int t = threadIdx.x; t < nseg * HP; t += NTH) {
        sm_ms[t] = coherent_load(&p.ws_ml[(slot0 + t) * 2]);
        sm_a[t] = coherent_load(&p.ws_ml[(slot0 + t) * 2 + 1]);
    }
    __syncthreads();
    if (threadIdx.x < HP) {
        const int h = threadIdx.x;
        float M = kNegInf;
        for (int k = 0; k < nseg; ++k) M = fmaxf(M, sm_ms[k * HP + h]);
        float lsum = 0.0f;
        for (int k = 0; k < nseg; ++k) {
            const float a = fast_exp2(sm_ms[k * HP + h] - M);
            lsum += a * sm_a[k * HP + h];
            sm_a[k * HP + h] = a;
        }
        sm_ls[h] = 1.0f / lsum;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < HP * D; idx += NTH) {
        const int h = idx / D;
        const int d = idx - h * D;
        if (h >= heads_here) continue;
        float o = 0.0f;
        int k = 0;
        for (; k + 4 <= nseg; k += 4) {
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = coherent_load(&p.ws_o[(slot0 + (size_t)(k + q) * HP + h) * D + d]);
#pragma unroll
            for (int q = 0; q < 4; ++q) o += sm_a[(k + q) * HP + h] * v[q];
        }
        for (; k < nseg; ++k) o += sm_a[k * HP + h] * coherent_load(&p.ws_o[(slot0 + (size_t)k * HP + h) * D + d]);
        A::st(p.out, ((size_t)b * p.H + h0 + h) * D + d, o * sm_ls[h]);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&p.counters[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
constexpr int kGqaBlocksPerCu = 1;   // target pieces per CU (one 8-wave workgroup: about 83 KiB of LDS)

template <int KV, int D, int HP, bool PG>
hipError_t launch_gqa_t(const Params& p, hipStream_t s) {
    hipLaunchKernelGGL((gqa_kernel<KV, D, HP, kGqaWaves, PG>), dim3(p.S), dim3(64 * kGqaWaves), 0, s, p);
    return hipGetLastError();
}

template <int KV, int D, int GT, bool PG>
hipError_t launch_attention_t(const Params& p, int nw, hipStream_t s) {
    dim3 grid(p.S, p.Hkv * p.n_hg, p.B);
    if constexpr ((KV == KV_F16 || KV == KV_BF16) && (GT == 4 || GT == 8)) {
        if (p.balanced) return launch_gqa_t<KV, D, GT, PG>(p, s);
    }
    constexpr int U = unroll_for(GT);
    if constexpr (wide_built(KV, GT)) {
        if (nw == 16) {
            hipLaunchKernelGGL((attention_kernel<KV, D, GT, U, 16, PG>), grid, dim3(64 * 16), 0, s, p);
            return hipGetLastError();
        }
    }
    if (nw != 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attention_kernel<KV, D, GT, U, 4, PG>), grid, dim3(64 * 4), 0, s, p);
    return hipGetLastError();
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
    const char* e = std::getenv("FTM_GQA_BLOCKS_PER_CU");
    const int v = e ? std::atoi(e) : 0;
    return v > 0 && v <= 16 ? v : kGqaBlocksPerCu;
}

bool use_gqa_mfma(int kv, int gtile, int batch) {
    if (!((kv == KV_F16 || kv == KV_BF16) && (gtile == 4 || gtile == 8))) return false;
    if (batch > kGqaMaxBatch) return false;
    const char* e = std::getenv("FTM_GQA_VALU");
    return !(e && *e == '1');
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
