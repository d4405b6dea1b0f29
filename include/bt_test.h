/*
 * bt_test.h — diagnostic entry points of libbt for tests and benchmarks.
 * They are not needed to run inference; see bt.h for the inference API.
 */
#ifndef BT_TEST_H_
#define BT_TEST_H_

#include <stddef.h>
#include <stdint.h>

#include "bt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel classes timed by the profiler (BT_PROFILE_KINDS of them): 0 embedder gathers and
 * start-slot rows, 1 LayerNorms, 2 [q|k|v|up] GEMMs (with GELU), 3 [out|down] GEMMs (residual
 * add), 4 context projection (and the cross-attention key/value projection), 5 classifier +
 * argmax, 6 prefill attention, 7 prefill rotary/KV scatter, 8 block-attention decode (incl. split
 * merge), 9 local attention, 10 greedy-id finalisation, 11 cross-attention, 12 local attention
 * inside the [out|down] GEMM (token decoder, one new slot per row).  Each class is counted
 * separately for launches made by bt_prefill (index k) and by bt_decode_step (index 13 + k). */
#define BT_PROFILE_KINDS 13

/* Start (on != 0) or stop recording a pair of HIP events around every kernel launch of the
 * handle, on the handle's stream.  Clears what was recorded before. */
int bt_profile_enable(bt_handle* h, int32_t on);

/* Synchronise the handle's stream and return, for each of the 2 * BT_PROFILE_KINDS classes (n_kinds
 * must be at least that), the summed event time in ms, the number of launches, and the summed
 * algorithmic bytes and flops of those launches (the minimal traffic and arithmetic of each
 * operation: weights and KV read once, activations read and written once).  Then clear the record. */
int bt_profile_read(bt_handle* h, int32_t n_kinds, double* total_ms, int64_t* launches, double* bytes,
                    double* flops);

/* Launch again, `reps` times back to back on the handle's stream, the kernel of one decode launch
 * class at the batch of the last prefill, for timing it without per-launch events.  kind (profile
 * class index): 2 = the decode [q|k|v|up] GEMM, cycling over the weights of all token- and
 * block-decoder layers and over up to 64 row ranges of the LayerNorm outputs (operands not left in a
 * cache by the previous launch); 8 = block-attention decode at the current block-KV length, cycling over
 * the block-decoder layers; 12 = the token decoder's local attention inside its [out|down] GEMM
 * (see bt_test_fuse_local) at the next local slot, cycling over the token-decoder layers
 * (BT_ERR_UNSUPPORTED where decode steps do not run it); -1 = an empty kernel of 256 workgroups of
 * 256 threads, whose back-to-back launches time the fixed cost of one dependent launch on the stream
 * (the floor under the duration of every decode launch).  Only activations and split-K partials
 * are overwritten, plus the cache entry each kind appends (kind 8: the block-KV entry at the
 * current length; kind 12: the local-KV entry at the next local slot), which is not yet valid and is
 * written again by the next step that uses it, so decoding can continue afterwards.
 * BT_ERR_STATE before a prefill; BT_ERR_INVALID_ARG for other kinds. */
int bt_test_replay(bt_handle* h, int32_t kind, int32_t reps);

/* enable = 0: decode steps launch the token decoder's local attention (and, with cross-attention
 * injection, the cross-attention) separately from its [out|down] GEMM instead of inside it (the
 * default where the shape allows: fp16, head width 64, at most 256 rows).  Same results up to the summation order of the
 * residual update.  Drops captured decode graphs when the setting changes. */
int bt_test_fuse_local(bt_handle* h, int32_t enable);

/* C[M][N] = scale * A[M][K] * W[N][K]^T in fp32 (C row-major), on `stream` (a hipStream_t).
 * dtype BT_FP32: A and W fp32, row-major.  BT_BF16: A and W fp16 (the library's matrix-operand
 * type) in the library's operand order, K % 64 == 0, N % 32 == 0: a matrix with R rows (R rounded up
 * to a multiple of 16; A holds ceil(M / 16) * 16 * K elements) is stored as the 16 x 32 tiles
 * (g, s) = (rows 16g.., columns 32s..) in the order g-major, s-minor, 512 elements each; inside a
 * tile, the 8 elements (row 16g + r, columns 32s + 8q .. 32s + 8q + 7) sit at element 8 * (16q + r).
 * Device pointers; synchronous errors only. */
int bt_test_gemm(int32_t dtype, const void* d_a, const void* d_w, float* d_c, int32_t M, int32_t N, int32_t K,
                 float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BT_TEST_H_ */
