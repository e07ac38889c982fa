// prefill.hip -- gfx950 kernels for prefill: the whole prompt of every
// sequence in one step.  The prompt is processed in parallel where decode
// goes token by token ([lpnh.cn/news/2765398] section 1.1): its K/V rows
// are appended to the cache, and every position t attends causally to
// positions [0, t] of its KV head.
//
// prefill_append_kernel: the prompt's K/V rows, with the bias added in fp32,
//   rounded to nearest even into the cache (one 16-byte slice per thread).
// prefill_attn_kernel: one workgroup of 4 waves owns 64 query positions of
//   one query head; wave w owns 16 of them.  The workgroup streams the key
//   positions [0, last query] in tiles of 64 through LDS; each wave computes,
//   32 keys at a time (four independent accumulation chains), S^T = K Q^T
//   for 16 keys x its 16 queries and O += P V on the matrix cores
//   (v_mfma_f32_16x16x32 and 16x16x16), with the online softmax in between
//   and the causal mask on the diagonal tiles.  S^T leaves each lane with
//   four consecutive keys of one query, which is the A-operand layout of P;
//   V is read down its columns with the transposing LDS read.  The query
//   (bias added, log2(e)/sqrt(D) folded in, kept in registers) and the
//   weights enter as hi/lo
//   halves, so about 16 (bf16) or 22 (fp16) bits of each reach the fp32
//   accumulators, as in the decode pass.  Workgroups with the most keys
//   are launched first.
#include <cstdlib>

#include "gfx950.hpp"

namespace ftm {
namespace {

constexpr int kPQ = 64;                   // query positions per workgroup (16 per wave)
constexpr int kPK = 64;                   // key positions per LDS tile
constexpr float kNegInfP = -__builtin_inff();

template <int KV, int D>
__global__ void __launch_bounds__(256) prefill_append_kernel(const PrefillParams p) {
    constexpr int EPL = 8;                  // elements per thread (16 bytes)
    constexpr int SL = D / EPL;             // slices per row
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t per_seq = (size_t)p.S * p.Hkv * SL;
    if (idx >= (size_t)p.B * per_seq) return;
    const int b = (int)(idx / per_seq);
    const size_t rem = idx - (size_t)b * per_seq;
    const int t = (int)(rem / ((size_t)p.Hkv * SL));
    const int j = (int)(rem / SL % p.Hkv);
    const int c = (int)(rem % SL);
    const int Sb = p.seq_lens ? p.seq_lens[b] : p.S;
    if (Sb < 1 || Sb > p.S || t >= Sb) return;         // invalid length: no append
    const size_t src = (((size_t)b * p.S + t) * p.Hkv + j) * D + c * EPL;
    const size_t dst = (((size_t)b * p.Hkv + j) * p.Lmax + t) * D + c * EPL;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const void* in = which ? p.v_new : p.k_new;
        void* cache = which ? p.v_cache : p.k_cache;
        const u32x4 raw = *(const u32x4*)((const uint16_t*)in + src);
        uint32_t hb[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint32_t bits = (raw[e / 2] >> (16 * (e % 2))) & 0xffffu;
            float x = KV == KV_F16 ? half_bits_to_float(bits) : bf16_bits_to_float(bits);
            if (p.bias) {
                const uint32_t bb = ((const uint16_t*)p.bias)[(size_t)(p.H + which * p.Hkv + j) * D + c * EPL + e];
                x = x + (KV == KV_F16 ? half_bits_to_float(bb) : bf16_bits_to_float(bb));   // one fp32 rounding
            }
            hb[e] = KV == KV_F16 ? float_to_half_bits(x) : float_to_bf16_bits(x);
        }
        *(u32x4*)((uint16_t*)cache + dst) = u32x4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16),
                                                  hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
    }
}

template <int KV, int D>
__global__ void __launch_bounds__(256) prefill_attn_kernel(const PrefillParams p) {
    using MF = Mfma<KV>;
    typedef typename MF::vec8 vec8;
    typedef typename MF::vec4 vec4;
    constexpr int ROW = D * 2;
    constexpr int KPITCH = ROW + 16;        // 16-byte reads of 16 rows hit distinct banks
    constexpr int VPITCH = ROW + 32;        // transposing reads of 4 rows x 32 bytes hit distinct banks
    constexpr int KK = D / 32;              // S^T: MFMA steps over the head dim
    constexpr int DT = D / 16;              // O: 16-column tiles
    constexpr int LPR = D / 8;              // tile loads: lanes per row (16 bytes each)
    constexpr int RPI = 256 / LPR;          // tile loads: rows per workgroup-wide load
    constexpr int NLD = kPK / RPI;          // tile loads per thread per tile, each of K and V
    // K and V tiles; before the first tile the same memory stages the query
    // operand, which the waves then keep in registers
    constexpr int QBYTES = 2 * 16 * KPITCH;
    static_assert(4 * QBYTES <= kPK * (KPITCH + VPITCH), "query staging fits in the tiles");
    __shared__ __attribute__((aligned(16))) unsigned char smem[kPK * (KPITCH + VPITCH)];
    unsigned char* ktile = smem;
    unsigned char* vtile = smem + kPK * KPITCH;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;                // MFMA layout: k group / key quad
    const int n = lane & 15;                // MFMA layout: key row (A) / query column (B, C)
    const int b = blockIdx.z;
    const int h = blockIdx.y;
    const int j = h / (p.H / p.Hkv);
    const int qblk = gridDim.x - 1 - blockIdx.x;   // the blocks with the most keys first
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
    const int kend = min(t0 + kPQ, Sb);     // keys [0, kend) are needed
    const int tq = t0 + wave * 16;          // this wave's first query

    // query operand of S^T for this wave's 16 queries: hi and lo halves of
    // (q + b_q) * log2(e) / sqrt(D); queries past the prompt are zero
    {
        unsigned char* qb = smem + wave * QBYTES;
#pragma unroll
        for (int r = 0; r < 16 / (64 / LPR); ++r) {
            const int row = r * (64 / LPR) + lane / LPR;
            const int pc = lane % LPR;
            const int t = tq + row;
            float x[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            if (t < Sb) {
                const u32x4 raw = *(const u32x4*)((const uint16_t*)p.q + (((size_t)b * p.S + t) * p.H + h) * D + pc * 8);
                Elem16<KV>::unpack(raw, x);
                if (p.bias) {
                    float bx[8];
                    Elem16<KV>::unpack(*(const u32x4*)((const uint16_t*)p.bias + (size_t)h * D + pc * 8), bx);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = x[e] + bx[e];
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= p.qscale;
            }
            vec8 hi, lo;
            MF::split8(x, hi, lo);
            *(vec8*)(qb + row * KPITCH + pc * 16) = hi;
            *(vec8*)(qb + 16 * KPITCH + row * KPITCH + pc * 16) = lo;
        }
    }

    // K/V rows [0, kend) of (b, j) from the cache; rows past kend read as zero
    const size_t row0 = ((size_t)b * p.Hkv + j) * p.Lmax;
    const auto krs = make_rsrc((const char*)p.k_cache + row0 * ROW, (uint32_t)kend * ROW);
    const auto vrs = make_rsrc((const char*)p.v_cache + row0 * ROW, (uint32_t)kend * ROW);
    const int lr = tid / LPR, lc = tid % LPR;
    u32x4 kr[NLD], vr[NLD];
    auto issue = [&](int k0) {
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int off = (k0 + u * RPI + lr) * ROW + lc * 16;
            kr[u] = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, 0);
            vr[u] = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
        }
    };
    issue(0);

    float m = kNegInfP;                     // query n: running max (same in all four quads)
    float l = 0.0f;                         // query n: this lane's share of the sum
    f32x4 acc[DT];                          // O[query 4g+i][16 tn + n]
#pragma unroll
    for (int tn = 0; tn < DT; ++tn) acc[tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // the query operand stays in registers: B operand of step kk, hi and lo
    vec8 qh[KK], ql[KK];
    {
        const unsigned char* qb = smem + wave * QBYTES;
        lds_wave_fence();
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int piece = (kk * 4 + g) * 16;
            qh[kk] = MF::bits8(*(const u32x4*)(qb + n * KPITCH + piece));
            ql[kk] = MF::bits8(*(const u32x4*)(qb + 16 * KPITCH + n * KPITCH + piece));
        }
    }

    for (int k0 = 0; k0 < kend; k0 += kPK) {
        __syncthreads();                    // the previous tile is consumed
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            *(u32x4*)(ktile + (u * RPI + lr) * KPITCH + lc * 16) = kr[u];
            *(u32x4*)(vtile + (u * RPI + lr) * VPITCH + lc * 16) = vr[u];
        }
        __syncthreads();
        if (k0 + kPK < kend) issue(k0 + kPK);
        __builtin_amdgcn_sched_barrier(0);
        // two 16-key sub-tiles per step: four independent accumulation chains
#pragma unroll
        for (int sp = 0; sp < kPK / 32; ++sp) {
            const int kb = k0 + 32 * sp;    // first key of the pair
            if (kb > tq + 15) break;        // every key after every query of this wave
            // S^T: row = key kb + 16 h2 + 4g + i, column = query tq + n
            f32x4 sh[2], sl[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) sh[h2] = sl[h2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int piece = (kk * 4 + g) * 16;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const vec8 ka = MF::bits8(*(const u32x4*)(ktile + (32 * sp + 16 * h2 + n) * KPITCH + piece));
                    sh[h2] = MF::mma32(ka, qh[kk], sh[h2]);
                    sl[h2] = MF::mma32(ka, ql[kk], sl[h2]);
                }
            }
            // causal mask (and keys past the prompt, which lie after every valid query)
            float s[2][4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s[h2][i] = kb + 16 * h2 + 4 * g + i <= tq + n ? sh[h2][i] + sl[h2][i] : kNegInfP;
            float mt = kNegInfP;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[h2][i]);
            mt = fmaxf(mt, __shfl_xor(mt, 16));
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float mn = fmaxf(m, mt);
            const float ms = mn == kNegInfP ? 0.0f : mn;
            const float alpha = fast_exp2(m - ms);
            m = mn;
            float ls = 0.0f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s[h2][i] = fast_exp2(s[h2][i] - ms);
                    ls += s[h2][i];
                }
            l = l * alpha + ls;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
                for (int tn = 0; tn < DT; ++tn) acc[tn][i] *= ai;
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                vec4 ph, pl;
                MF::split4(s[h2], ph, pl);
                // B operand V[key 4g+i][16 tn + n]: lane n of group g names row
                // 4g + n/4 of the sub-tile, columns 4(n%4)..+3
                const unsigned char* vrow = vtile + (32 * sp + 16 * h2 + 4 * g + (n >> 2)) * VPITCH + (n & 3) * 8;
#pragma unroll
                for (int tn = 0; tn < DT; ++tn) {
                    const s16x4 tv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4*)(vrow + tn * 32));
                    const vec4 vb = __builtin_bit_cast(vec4, tv);
                    acc[tn] = MF::mma16(ph, vb, acc[tn]);
                    acc[tn] = MF::mma16(pl, vb, acc[tn]);
                }
            }
        }
    }

    // l over the four quads of the column; out = O / l, rows 4g + i
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tq + 4 * g + i;
        const float inv = 1.0f / __shfl(l, 4 * g + i);
        if (t < Sb) {
            const size_t o = (((size_t)b * p.S + t) * p.H + h) * D;
#pragma unroll
            for (int tn = 0; tn < DT; ++tn) {
                const float v = acc[tn][i] * inv;
                ((uint16_t*)p.out)[o + tn * 16 + n] =
                    (uint16_t)(KV == KV_F16 ? float_to_half_bits(v) : float_to_bf16_bits(v));
            }
        }
    }
}

template <int KV, int D>
hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
    const size_t slices = (size_t)p.B * p.S * p.Hkv * (D / 8);
    hipLaunchKernelGGL((prefill_append_kernel<KV, D>), dim3((unsigned)((slices + 255) / 256)), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((p.S + kPQ - 1) / kPQ, p.H, p.B);
    hipLaunchKernelGGL((prefill_attn_kernel<KV, D>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int kv, int head_dim, hipStream_t s) {
    if (kv == KV_F16) return head_dim == 64 ? launch_prefill_t<KV_F16, 64>(p, s) : launch_prefill_t<KV_F16, 128>(p, s);
    if (kv == KV_BF16) return head_dim == 64 ? launch_prefill_t<KV_BF16, 64>(p, s) : launch_prefill_t<KV_BF16, 128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace ftm
