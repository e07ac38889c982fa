// qkv_proj.hip -- gfx950 kernel for the fused QKV projection of a decode
// step: y = x W^T (+ bias) for x [B, hidden] and W [(H + 2 Hkv) D, hidden],
// written straight into the q [B, H, D], k_new [B, Hkv, D] and v_new
// [B, Hkv, D] layouts the attention reads ([lpnh.cn/news/2765398] section
// 2.1: Q, K and V come out of one projection and are split three ways with
// no extra round trip through memory).
//
// At decode batch sizes (B <= 64) the product reads every weight once and
// does at most 64 multiply-adds per weight: it is bound by the HBM stream
// of W, so the design streams W exactly once, coalesced, and keeps the
// arithmetic on the matrix cores out of its way.
//
// One workgroup (8 waves) owns 16 FT output features over the whole hidden
// dimension, split in eight: wave w takes an eighth of the k range.  Per
// iteration a wave loads 8 KiB of its weight rows (each load instruction
// covers whole 128-512-byte row segments), stages them in LDS and reads
// them back in the B-operand layout of v_mfma_f32_16x16x32.  x, small and
// read by every workgroup from L2, comes in the A-operand layout directly
// (16 rows x 64 bytes per load) or, with four column tiles and more than 16
// rows, in whole 128-byte lines through a per-wave LDS tile; each load
// serves FT products.  The next iteration's loads are in flight while the
// matrix cores work.  The eight partial sums meet in LDS in a fixed order,
// the bias is added in fp32, and the result is rounded to nearest even.
// Large batches with fewer column tiles take the k-split kernel below.
#include <cstdlib>

#include "gfx950.hpp"

namespace ftm {
namespace {

constexpr int kWaves = 8;                 // the k range is split across the waves of a workgroup
constexpr int kStream = 2;                // non-temporal: every weight is read once

// The activation type's matrix-core product on 16-byte operands, and its
// scalar load and round-to-nearest-even store.
template <int ACT> struct QMma {
    using MF = Mfma<ACT>;
    __device__ static f32x4 mma(const u32x4 a, const u32x4 b, const f32x4 c) {
        return MF::mma32(MF::bits8(a), MF::bits8(b), c);
    }
    __device__ static float ld(const void* p, size_t i) {
        const uint32_t h = ((const uint16_t*)p)[i];
        return ACT == KV_F16 ? half_bits_to_float(h) : bf16_bits_to_float(h);
    }
    __device__ static void st(void* p, size_t i, float v) {
        ((uint16_t*)p)[i] = (uint16_t)(ACT == KV_F16 ? float_to_half_bits(v) : float_to_bf16_bits(v));
    }
};

// MT: batch tiles of 16 rows (B <= 16 MT).  FT: 16-feature column tiles
// per workgroup, each wave computing all of them over its k range, so that
// one load of x serves FT products (FT = MT keeps the bytes of x read per
// weight byte at one).  A wave iteration covers KIT = 256 / FT k (8 KiB of
// weights in 8 loads) for FT = 1, 2, 4, and KIT = 128 for FT = 3 (12 KiB in
// 12 loads).  The last workgroup may hold fewer than 16 FT features: its
// weight rows past the end read as zero and its tiles past the end are not
// written.
template <int ACT, int MT, int FT, bool XS>
__global__ void __launch_bounds__(64 * kWaves) qkv_proj_kernel(const QkvParams p) {
    using M = QMma<ACT>;
    constexpr int COLS = 16 * FT;           // output features per workgroup
    constexpr int KIT = FT == 3 ? 128 : 256 / FT;   // k per wave iteration
    constexpr int KS = KIT / 32;            // MFMA k-steps per iteration
    constexpr int PITCH = KIT * 2 + 16;     // LDS row pitch: 16-byte reads of 16 rows hit distinct banks
    constexpr int LPRW = KIT / 8;           // weight loads: lanes per row (16 bytes each)
    constexpr int RPIW = 64 / LPRW;         // weight loads: rows per instruction
    constexpr int NLD = COLS / RPIW;        // weight loads per iteration
    static_assert(NLD * RPIW == COLS, "the loads cover the workgroup's rows");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;                // MFMA operands: k group
    const int n = lane & 15;                // MFMA operands: batch row (A), feature (B)
    const int lrow = lane / LPRW;           // weight loads: row within an instruction's rows
    const int lcol = lane % LPRW;           // weight loads: 16-byte chunk within the row
    const int f0 = blockIdx.x * COLS;
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    const int nit = p.hidden / KIT;
    const int it0 = wave * nit / kWaves;
    const int it1 = (wave + 1) * nit / kWaves;
    const uint32_t row_bytes = (uint32_t)p.hidden * 2;
    // the workgroup's weight rows; x rows past the batch read as zero
    const auto wrs = make_rsrc((const char*)p.w + (size_t)f0 * row_bytes, (uint32_t)min(COLS, n_out - f0) * row_bytes);
    const auto xrs = make_rsrc(p.x, (uint32_t)p.B * row_bytes);

    // per-wave weight tiles (and, with XS, x tiles); after the loop, the
    // waves' partial sums (MT x FT tiles each)
    constexpr int TILE = COLS * PITCH;
    constexpr int XTILE = XS ? 16 * MT * PITCH : 0;
    constexpr int RED = kWaves * MT * FT * 64 * 16;
    constexpr int WAVE_LDS = TILE + XTILE;
    __shared__ __attribute__((aligned(16))) unsigned char smem[WAVE_LDS * kWaves > RED ? WAVE_LDS * kWaves : RED];
    unsigned char* tile = smem + wave * WAVE_LDS;
    unsigned char* xtile = tile + TILE;
    // XS: x comes in whole 128-byte lines (XL lanes per row of KIT k, XR
    // rows per instruction), is written to the wave's x tile and read back
    // in the A-operand layout
    constexpr int XL = KIT * 2 / 16;
    constexpr int XR = 64 / XL;
    constexpr int NX = 16 * MT / XR;
    static_assert(!XS || NX * XR == 16 * MT, "the x loads cover the batch tiles");

    // iterations outside [it0, it1) take an offset past the descriptor's
    // range: their loads fetch nothing, so the prefetch needs no branch
    // (a branch around it makes the compiler wait for every load in flight)
    u32x4 wr[NLD];
    auto issue_w = [&](int it) {
        const uint32_t koff = it < it1 ? (uint32_t)it * (KIT * 2) : 0x40000000u;
#pragma unroll
        for (int u = 0; u < NLD; ++u)
            wr[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (RPIW * u + lrow) * row_bytes + koff + lcol * 16,
                                                          0, kStream);
    };
    // XS: x of the next iteration in whole lines, in flight with its weights
    u32x4 xl[XS ? NX : 1];
    auto issue_x = [&](int it) {
        const uint32_t koff = it < it1 ? (uint32_t)it * (KIT * 2) : 0x40000000u;
#pragma unroll
        for (int u = 0; u < NX; ++u)
            xl[u] = __builtin_amdgcn_raw_buffer_load_b128(xrs, (XR * u + lane / XL) * row_bytes + koff + (lane % XL) * 16,
                                                          0, 0);
    };
    f32x4 acc[MT][FT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) acc[mt][ft] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    issue_w(it0);
    if constexpr (XS) issue_x(it0);
    __builtin_amdgcn_sched_barrier(0);
    for (int it = it0; it < it1; ++it) {
        // this iteration's x (A operand: batch row 16 mt + n, k = 32 s + 8 g ..),
        // issued after the weights of this iteration and before those of the next
        u32x4 xr[MT][KS];
        if constexpr (!XS) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    xr[mt][s] = __builtin_amdgcn_raw_buffer_load_b128(
                        xrs, (16 * mt + n) * row_bytes + (it * KIT + 32 * s + 8 * g) * 2, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // stage this iteration's weights, then send the next iteration's out
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < NLD; ++u) *(u32x4*)(tile + (RPIW * u + lrow) * PITCH + lcol * 16) = wr[u];
        if constexpr (XS) {
#pragma unroll
            for (int u = 0; u < NX; ++u) *(u32x4*)(xtile + (XR * u + lane / XL) * PITCH + (lane % XL) * 16) = xl[u];
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_w(it + 1);
        if constexpr (XS) issue_x(it + 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (XS) {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    xr[mt][s] = *(const u32x4*)(xtile + (16 * mt + n) * PITCH + (32 * s + 8 * g) * 2);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // B operand: feature 16 ft + n, k = 32 s + 8 g ..
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int ft = 0; ft < FT; ++ft) {
                const u32x4 wb = *(const u32x4*)(tile + (16 * ft + n) * PITCH + (32 * s + 8 * g) * 2);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][ft] = M::mma(xr[mt][s], wb, acc[mt][ft]);
            }
        }
    }

    // the eight partial sums meet in LDS: every wave writes its tiles, then
    // wave w adds up tiles w, w + 8, ... over the waves in order (a fixed
    // order: the result is deterministic), adds the bias and writes them
    f32x4* red = (f32x4*)smem;              // [kWaves][MT][FT][64]
    auto slot = [&](int w, int mt, int ft) { return red + ((w * MT + mt) * FT + ft) * 64 + lane; };
    __syncthreads();                        // the tiles are free
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) *slot(wave, mt, ft) = acc[mt][ft];
    __syncthreads();

    // C layout: lane (g, n) holds feature f0 + 16 ft + n for batch rows
    // 16 mt + 4 g + i.  Column tiles never straddle the Q/K/V boundaries
    // (H D and Hkv D are multiples of 16).
    const int qd = p.H * p.D, kd = p.Hkv * p.D;
    for (int t = wave; t < MT * FT; t += kWaves) {
        const int mt = t / FT, ft = t - mt * FT;
        const int f = f0 + 16 * ft + n;
        const int fb = f0 + 16 * ft;        // the tile's first feature, the same in every lane
        if (fb >= n_out) continue;          // past the last feature (n_out is a multiple of 16)
        f32x4 sum = *slot(0, mt, ft);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) sum += *slot(w, mt, ft);
        void* dst;
        int width, col;
        if (fb < qd) {
            dst = p.q, width = qd, col = f;
        } else if (fb < qd + kd) {
            dst = p.k_new, width = kd, col = f - qd;
        } else {
            dst = p.v_new, width = kd, col = f - qd - kd;
        }
        const float bf = p.bias ? M::ld(p.bias, f) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * g + i;
            if (row < p.B) M::st(dst, (size_t)row * width + col, p.bias ? sum[i] + bf : sum[i]);
        }
    }
}

// Batches above 32 rows: x is then about as large as a 48- or 64-feature
// slice of the weights, and every workgroup of the one-pass kernel reads
// all of it from L2, which costs time on top of the weight stream (at 64
// rows and 64 features per workgroup, 8.6 us of 37).  This variant gives a
// workgroup 128 features over 1/KSPLIT of the hidden dimension (KSPLIT
// workgroups per column, enough to cover the CUs), halving x per weight
// byte: every wave
// owns 16 features, and per iteration the workgroup loads one x tile of
// KIT k into LDS, shared by all eight waves (double-buffered, one barrier
// per iteration).  Each workgroup writes its fp32 partial through to the
// device coherence point and bumps its column's count; the workgroup that
// completes the count adds the KSPLIT partials in split order (the sum does
// not depend on which one finished last), adds the bias and writes q, k_new
// and v_new.
constexpr int kSplitKit = 256;          // k per iteration: whole 512-byte row segments
constexpr int kSplitCols = 16 * kWaves; // features per workgroup
constexpr int kCoherent = 16;           // cache policy sc1: agent-scope coherent access

template <int ACT, int MT>
__global__ void __launch_bounds__(64 * kWaves) qkv_split_kernel(const QkvParams p, const int ksplit) {
    using M = QMma<ACT>;
    constexpr int KIT = kSplitKit;
    constexpr int KS = KIT / 32;            // MFMA k-steps per iteration
    constexpr int PITCH = KIT * 2 + 16;     // LDS row pitch: 16-byte reads of 16 rows hit distinct banks
    constexpr int LPR = KIT / 8;            // loads: lanes per row (16 bytes each)
    constexpr int RPI = 64 / LPR;           // loads: rows per instruction
    constexpr int NLD = 16 / RPI;           // weight loads per wave and iteration (16 rows)
    constexpr int XROWS = 16 * MT;          // x rows staged (rows past the batch read as zero)
    constexpr int NXL = XROWS / kWaves / RPI;   // x loads per wave and iteration
    static_assert(NXL * RPI * kWaves == XROWS, "the waves' x loads cover the tile");
    constexpr int XTILE = XROWS * PITCH;
    constexpr int WTILE = 16 * PITCH;
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * XTILE + kWaves * WTILE];
    __shared__ int sm_last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int n = lane & 15;
    const int lrow = lane / LPR;
    const int lcol = lane % LPR;
    const int col = blockIdx.x / ksplit;
    const int kh = blockIdx.x - col * ksplit;
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    const int f0 = col * kSplitCols + 16 * wave;    // the wave's first feature
    const int nit = p.hidden / KIT;
    const int it0 = kh * nit / ksplit;
    const int it1 = (kh + 1) * nit / ksplit;
    const uint32_t row_bytes = (uint32_t)p.hidden * 2;
    // the wave's weight rows (none past the end: those read as zero)
    const auto wrs = make_rsrc((const char*)p.w + (size_t)min(f0, n_out) * row_bytes,
                               (uint32_t)max(0, min(16, n_out - f0)) * row_bytes);
    const auto xrs = make_rsrc(p.x, (uint32_t)p.B * row_bytes);
    unsigned char* wtile = smem + 2 * XTILE + wave * WTILE;

    // iterations past the range load from past the descriptors' ends:
    // nothing is fetched and no branch is needed
    u32x4 wr[NLD], xl[NXL];
    auto issue = [&](int it) {
        const uint32_t koff = it < it1 ? (uint32_t)it * (KIT * 2) : 0x40000000u;
#pragma unroll
        for (int u = 0; u < NLD; ++u)
            wr[u] = __builtin_amdgcn_raw_buffer_load_b128(wrs, (RPI * u + lrow) * row_bytes + koff + lcol * 16, 0,
                                                          kStream);
#pragma unroll
        for (int u = 0; u < NXL; ++u)
            xl[u] = __builtin_amdgcn_raw_buffer_load_b128(
                xrs, ((NXL * wave + u) * RPI + lrow) * row_bytes + koff + lcol * 16, 0, 0);
    };
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    issue(it0);
    __builtin_amdgcn_sched_barrier(0);
    for (int it = it0; it < it1; ++it) {
        unsigned char* xtile = smem + ((it - it0) & 1) * XTILE;
        // this iteration's tiles into LDS (the x tile whose readers were two
        // iterations back, past the last barrier), the next iteration's out
#pragma unroll
        for (int u = 0; u < NLD; ++u) *(u32x4*)(wtile + (RPI * u + lrow) * PITCH + lcol * 16) = wr[u];
#pragma unroll
        for (int u = 0; u < NXL; ++u)
            *(u32x4*)(xtile + ((NXL * wave + u) * RPI + lrow) * PITCH + lcol * 16) = xl[u];
        __builtin_amdgcn_sched_barrier(0);
        issue(it + 1);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();                    // every wave's part of the x tile is in
        // A operand: batch row 16 mt + n; B operand: feature f0 + n; k = 32 s + 8 g ..
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const u32x4 wb = *(const u32x4*)(wtile + n * PITCH + (32 * s + 8 * g) * 2);
            u32x4 xa[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xa[mt] = *(const u32x4*)(xtile + (16 * mt + n) * PITCH + (32 * s + 8 * g) * 2);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = M::mma(xa[mt], wb, acc[mt]);
        }
    }

    // partial of this workgroup: slot (col, kh), [wave][mt][lane] f32x4
    const size_t slot_f4 = (size_t)kWaves * MT * 64;
    const auto wsr = make_rsrc(p.ws + (size_t)col * ksplit * slot_f4 * 4, (uint32_t)(ksplit * slot_f4 * 16));
    auto at = [&](int k, int mt) { return (uint32_t)((((size_t)k * kWaves + wave) * MT + mt) * 64 + lane) * 16; };
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[mt]), wsr, at(kh, mt), 0, kCoherent);
    // the partial stores count as done only once the coherence point has
    // them; then the count goes up, and the workgroup that completes it
    // reads the others' partials with coherent loads
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        sm_last = __hip_atomic_fetch_add(&p.counters[col], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  ksplit - 1;
    __syncthreads();
    if (!sm_last) return;
    f32x4 sum[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sum[mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < ksplit; ++k) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 part = k == kh ? acc[mt]
                                       : __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                       wsr, at(k, mt), 0, kCoherent));
            sum[mt] = k == 0 ? part : sum[mt] + part;
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(&p.counters[col], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (f0 >= n_out) return;                // past the last feature (n_out is a multiple of 16)

    // C layout: lane (g, n) holds feature f0 + n for batch rows 16 mt + 4 g + i
    const int qd = p.H * p.D, kd = p.Hkv * p.D;
    const int f = f0 + n;
    void* dst;
    int width, c;
    if (f0 < qd) {
        dst = p.q, width = qd, c = f;
    } else if (f0 < qd + kd) {
        dst = p.k_new, width = kd, c = f - qd;
    } else {
        dst = p.v_new, width = kd, c = f - qd - kd;
    }
    const float bf = p.bias ? M::ld(p.bias, f) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * mt + 4 * g + i;
            if (row < p.B) M::st(dst, (size_t)row * width + c, p.bias ? sum[mt][i] + bf : sum[mt][i]);
        }
}

// Column tiles per workgroup.  Every CU streams weights at about the same
// rate, so the time goes with (rounds of workgroups over the CUs) x FT; the
// choice minimises that, and on a tie takes the larger FT (x read from L2
// fewer times).  On 256 CUs: four for 15360 features, three for 12288 and
// for 10240 (256 and 214 workgroups where four gave 192 and 160).
// FTM_QKV_COLUMN_TILES (1 to 4) forces the choice.
int column_tiles(int n_out, int n_cu) {
    const int forced = tuning().qkv_column_tiles;
    if (forced >= 1 && forced <= 4) return forced;
    int best = 4;
    long best_cost = -1;
    for (int ft = 4; ft >= 1; --ft) {
        const long wgs = (n_out + 16 * ft - 1) / (16 * ft);
        const long cost = (wgs + n_cu - 1) / n_cu * ft;
        if (best_cost < 0 || cost < best_cost) {
            best = ft;
            best_cost = cost;
        }
    }
    return best;
}

template <int ACT, int MT, int FT>
hipError_t launch_mf(const QkvParams& p, hipStream_t s) {
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    // x through LDS in whole lines where both tiles fit in LDS (four column
    // tiles) and x is large enough to matter (more than one batch tile)
    constexpr bool XS = FT == 4 && MT >= 2;
    hipLaunchKernelGGL((qkv_proj_kernel<ACT, MT, FT, XS>), dim3((n_out + 16 * FT - 1) / (16 * FT)), dim3(64 * kWaves),
                       0, s, p);
    return hipGetLastError();
}

template <int ACT, int MT>
hipError_t launch_m(const QkvParams& p, int ft, hipStream_t s) {
    switch (ft) {
    case 1: return launch_mf<ACT, MT, 1>(p, s);
    case 2: return launch_mf<ACT, MT, 2>(p, s);
    case 3: return launch_mf<ACT, MT, 3>(p, s);
    case 4: return launch_mf<ACT, MT, 4>(p, s);
    default: return hipErrorInvalidValue;
    }
}

// k-split workgroups per 128-feature column, or 1 (one pass).  The split
// serves batches above 32 rows where the one-pass kernel would take fewer
// than four column tiles: there x cannot be staged through LDS beside the
// weights and is read in the operand layout at a cost above the weights'
// (measured at batch 64, hidden 8192, 10240 features: 40 against 53 us).
// With four column tiles the one-pass kernel's barrier-free loop is the
// faster (37.0 against 38.4 us at 15360 features, hidden 5120).  The split
// count keeps the grid within the CUs, at most four, and at least two.  On
// 256 CUs: two for 12288 features, three for 10240.
// FTM_QKV_K_SPLIT (1 to 4) forces the choice.
int k_split(const QkvParams& p, int n_cu) {
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    const int nit = p.hidden / kSplitKit;
    const int cols = (n_out + kSplitCols - 1) / kSplitCols;
    const int forced = tuning().qkv_k_split;
    int ks;
    if (forced >= 1 && forced <= 4) {
        ks = forced;
    } else {
        if (p.B <= 32 || column_tiles(n_out, n_cu) == 4) return 1;
        ks = min(4, n_cu / cols);
    }
    ks = min(ks, nit);
    return ks >= 2 ? ks : 1;
}

template <int ACT, int MT>
hipError_t launch_split(const QkvParams& p, int ks, hipStream_t s) {
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    const int cols = (n_out + kSplitCols - 1) / kSplitCols;
    hipLaunchKernelGGL((qkv_split_kernel<ACT, MT>), dim3(cols * ks), dim3(64 * kWaves), 0, s, p, ks);
    return hipGetLastError();
}

template <int ACT>
hipError_t launch_t(const QkvParams& p, int n_cu, hipStream_t s) {
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    const int mt = (p.B + 15) / 16;
    const int ft = column_tiles(n_out, n_cu);
    if (p.hidden % 256 != 0 || n_out % 16 != 0) return hipErrorInvalidValue;
    const int ks = k_split(p, n_cu);
    if (ks > 1) {
        if (!p.ws || !p.counters) return hipErrorInvalidValue;
        switch (mt) {
        case 1: return launch_split<ACT, 1>(p, ks, s);
        case 2: return launch_split<ACT, 2>(p, ks, s);
        case 3: return launch_split<ACT, 3>(p, ks, s);
        case 4: return launch_split<ACT, 4>(p, ks, s);
        default: return hipErrorInvalidValue;
        }
    }
    switch (mt) {
    case 1: return launch_m<ACT, 1>(p, ft, s);
    case 2: return launch_m<ACT, 2>(p, ft, s);
    case 3: return launch_m<ACT, 3>(p, ft, s);
    case 4: return launch_m<ACT, 4>(p, ft, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t qkv_split_workspace(const QkvParams& p, int n_cu, size_t* n_counters) {
    const int ks = k_split(p, n_cu);
    const int n_out = (p.H + 2 * p.Hkv) * p.D;
    const size_t cols = (size_t)(n_out + kSplitCols - 1) / kSplitCols;
    *n_counters = ks > 1 ? cols : 0;
    return ks > 1 ? cols * ks * kWaves * ((p.B + 15) / 16) * 64 * 16 : 0;
}

hipError_t launch_qkv_proj(const QkvParams& p, int act, int n_cu, hipStream_t s) {
    switch (act) {
    case KV_F16: return launch_t<KV_F16>(p, n_cu, s);
    case KV_BF16: return launch_t<KV_BF16>(p, n_cu, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ftm
