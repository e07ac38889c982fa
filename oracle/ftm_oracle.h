/*
 * ftm_oracle.h -- plain, slow CPU reference for one decode step of masked
 * multi-head attention over a KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this.  It shares no code, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * What it computes, and where the pages say so (page address + section):
 *  - the QKV bias is added and Q/K/V are split three ways
 *      [lpnh.cn/news/2765398] section 2.1 (operator fusion of the QKV projection);
 *  - the new K/V row of every sequence is appended to a pre-allocated cache and
 *    only the current query attends to the cached rows
 *      [lpnh.cn/news/2765398] section 2.2; [intelliparadigm.com .../2131745]
 *      section 2.1 (cache filled position by position, layout [B,H,L,D]);
 *  - dot products, softmax with the maximum subtracted, weighted sum of V,
 *      [lpnh.cn/news/2765398] sections 2.1 and 6.1 (scaling against fp16
 *      overflow), [intelliparadigm.com .../2131745] section 6.2;
 *  - K/V stored as INT8 and converted back at compute time
 *      [pptc.cn/news/144085] section 3.1; [intelliparadigm.com .../2131745] 2.1;
 *  - query heads sharing K/V heads in groups (GQA)
 *      [pptc.cn/news/144085] section 3.4.
 * Where the pages leave a step open, the plainest reading is taken; every
 * such reading is listed in the design notes and in the comments below.
 *
 * Precision: attention arithmetic is in double.  The append is specified in
 * IEEE fp32 (add, divide, round-to-nearest-even) so that it is bit-exact.
 *
 * Parity pins: every function here is checked in tests/test_oracle_*.py
 * against closed forms, brute force and independent library routines.  The
 * accumulation order of any fast implementation is not pinned by the pages
 * (parity beyond the stated tolerances is unpinned).
 */
#ifndef FTM_ORACLE_H
#define FTM_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types, the oracle's own numbering. */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_I8 = 3 };

/* IEEE binary16 / bfloat16 bit patterns -> exact double. */
double orc_f16_bits_to_double(uint16_t bits);
double orc_bf16_bits_to_double(uint16_t bits);

/* fp32 -> binary16 / bfloat16, round to nearest, ties to even. */
uint16_t orc_float_to_f16_rne(float x);
uint16_t orc_float_to_bf16_rne(float x);

/* Quantise one row of n fp32 values to symmetric INT8:
 * scale = fl32(absmax / 127), code = clamp(rint(fl32(x / scale)), -127, 127),
 * all codes 0 when scale == 0.  Returns the scale. */
float orc_quantize_row_i8(const float* x, int n, int8_t* codes);

/* One decode step, all sequences.
 *   q        [B, H, D]          act dtype
 *   k_new    [B, Hkv, D]        act dtype
 *   v_new    [B, Hkv, D]        act dtype
 *   qkv_bias [(H + 2 Hkv) D]    act dtype, [b_q | b_k | b_v], may be NULL
 *   k_cache, v_cache [B, Hkv, Lmax, D] kv dtype, row L_b-1 written in place
 *   seq_lens [B] (NULL: every L_b = step); L_b counts the appended token
 *   kv_scales [2, B, Hkv, Lmax] fp32 (INT8 only), written in place
 *   out      [B, H, D] double
 *   probs    [B, H, step] double or NULL: softmax weights, zero past L_b
 * act dtype = kv dtype for float caches, fp16 for an INT8 cache.
 * A sequence with L_b outside [1, step] is left untouched and its out rows
 * are NaN.  n_threads <= 1 runs on the calling thread.
 * Returns 0, or -1 on an argument error. */
int orc_decode_mha(const void* q, const void* k_new, const void* v_new,
                   const void* qkv_bias, void* k_cache, void* v_cache,
                   const int32_t* seq_lens, int batch, int max_seq_len, int step,
                   int n_heads, int n_kv_heads, int head_dim, int kv_dtype,
                   float* kv_scales, double* out, double* probs, int n_threads);

#ifdef __cplusplus
}
#endif
#endif
