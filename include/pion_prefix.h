/*
 * pion_prefix.h - C ABI for attention over a resident, shared KV-cache prefix on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the ATTEND.PREFIX.* family of the "Shared KV Cache Serving" page
 * (section "Stage 2: ATTEND.PREFIX.* - Pion computes attention on cached K/V", Wire
 * forms) and of the "ATTEND.* and ATTEND.PREFIX.*" command page (Wire forms and the
 * externalized-attention command table). Argument order follows those wire forms
 * (sid, layer, H, N, D, ...); blobs become pointers.
 *
 * Conventions for every entry point:
 *   - Returns PION_OK (0) or a negative PION_ERR_* code; nothing throws across the ABI.
 *   - Arguments are validated before any GPU work is queued, so on an error no
 *     output is written.
 *   - Tensor pointers are DEVICE pointers (hipMalloc or a torch CUDA tensor on the
 *     same GPU), contiguous, in the layouts stated below. head_map is a HOST pointer.
 *   - Work is queued on `stream` (a hipStream_t passed as void*; NULL = the null
 *     stream) and is asynchronous: inputs must stay valid, and outputs must not be
 *     read, until `stream` has passed the call.
 *   - fp16 means IEEE binary16; out and lse are fp32.
 *   - The softmax scale is 1/sqrt(D); lse is the natural-log log-sum-exp of the
 *     scaled logits, so two partial results over disjoint key sets merge as
 *     lse = ln(e^lse1 + e^lse2), out = e^(lse1-lse) out1 + e^(lse2-lse) out2.
 *   - head_map: int32 per q-head naming its kv-head (GQA); NULL means
 *     h -> h / (H_q / H_kv), which requires H_kv to divide H_q.
 *   - Supported head dims: D in {32, 64, 96, 128, 160, 192, 256, 512} (the native SDPA
 *     head-dim set of the "Shared KV Cache Serving" page); other values ->
 *     PION_ERR_UNSUPPORTED. Batched-Q (M >= 32) fp16 queries run on matrix cores for
 *     every D but 512, which runs on the vector split kernel (same results).
 *   - Launch-plan limits: a query row is cut into at most 8192 key spans, and one query
 *     index's partials (H_q x spans x D fp32) must stay under 2^31 bytes; a query whose
 *     plan exceeds either returns PION_ERR_UNSUPPORTED before any launch (this happens
 *     only for token lists near 2^24 positions at H = 128, D = 512).
 *   - Calls are thread-safe (one library-wide lock guards the slot table).
 */
#ifndef PION_PREFIX_H
#define PION_PREFIX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The wire's "-ERR session not found" is PION_ERR_NOT_FOUND and its
 * "-COLDMISS" is PION_ERR_COLDMISS; +HIT/+COLD/+MISS are the 1/2/0 results of
 * pion_prefix_lookup (ATTEND.* page, ATTEND.PREFIX.LOOKUP row; "Shared KV Cache
 * Serving", Cold-tier state machine).
 *
 * Capacity and cold tier (same section). The slot table holds at most max_slots slots
 * and, when max_bytes > 0, at most max_bytes of resident K/V bytes (block-mean caches
 * not counted); defaults 4096 slots, no byte budget, 1024 cold entries (env
 * PION_MAX_SLOTS, PION_MAX_BYTES, PION_COLD_SLOTS at load; pion_prefix_set_capacity).
 * Every store and every successful query stamps its slot(s) with a logical clock. A
 * store that would exceed the capacity first demotes the least recently stamped slots
 * (never the key being stored): each one's device memory is released and its shape
 * moves to the cold registry (WARM -> COLD). When the registry overflows, its least
 * recently stamped entry is forgotten (MISSING). A query of a cold key returns
 * PION_ERR_COLDMISS and changes nothing; storing it again (from the caller's copy of
 * K/V) makes it warm and the most recent (COLD -> WARM, a rehydrate). Lookups, info and
 * failed queries stamp nothing. A device allocation failure also demotes, least
 * recently used first, before NOMEM is returned. Demotion frees memory that queued
 * work may still read only after that work has finished. */
enum {
    PION_OK = 0,
    PION_ERR_NOT_FOUND = -1,   /* no slot for (sid, layer), warm or cold */
    PION_ERR_INVALID = -2,     /* bad argument: null pointer, shape mismatch, range */
    PION_ERR_UNSUPPORTED = -3, /* valid request the library does not implement (D, ...) */
    PION_ERR_NOMEM = -4,       /* device memory short with nothing left to demote, or
                                  a slot larger than the byte budget */
    PION_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed */
    PION_ERR_COLDMISS = -6,    /* the key was demoted to the cold tier: store it again */
    PION_ERR_SCRATCH = -7      /* pion_prefix_query_noalloc: the call needs more scratch
                                  than the fixed area holds (nothing was launched) */
};

/* Resident formats. FP16 keeps K and V as given. MLX4G32 is the int4 group-32 affine
 * tier ("Shared KV Cache Serving", Quantized tier - mlx4g32; V-store page, The
 * mlx4g32 tier), quantized on the device at store time with pion_kv_quantize_mlx4g32.
 * FP32 keeps fp32 K and V (the sdpa_*_fp32 kernels of the native SDPA paragraph).
 *
 * Precision of the arrays a call passes: on an FP32 slot, K and V of the store, Q of
 * every query form and the suffix K_suf, V_suf are fp32; on FP16 and MLX4G32 slots they
 * are fp16. out and lse are fp32 always. An FP32 slot runs every query form on the
 * vector split kernel (no fp16 matrix-core rounding of its values). */
enum { PION_KV_FP16 = 0, PION_KV_MLX4G32 = 1, PION_KV_FP32 = 2 };

/* ATTEND.PREFIX.STORE <sid> <layer> <H> <N> <D> <K_blob> <V_blob>.
 * Copies K and V, [H, N, D] each (fp16, or fp32 for PION_KV_FP32), into a library-owned slot keyed (sid, layer)
 * and keeps them resident until pion_prefix_drop, demotion (see Capacity above) or
 * library unload (the command table: "resident until DROP"). Storing a live key
 * replaces its slot and drops any cached block means; storing a cold key rehydrates it. The library owns the slot memory; K and V may be freed once
 * `stream` has passed the call. sid is a NUL-terminated string of 1..255 bytes.
 * Errors: INVALID (null/empty sid, H/N/D <= 0, H > 255, kv_format unknown, D % 32 != 0
 * for MLX4G32), UNSUPPORTED (D; MLX4G32 with N * D >= 2^33), NOMEM (larger than the
 * byte budget, or device memory short with nothing left to demote; a cold key stays
 * cold), HIP. */
int pion_prefix_store(const char *sid, int layer, int H, int N, int D,
                      const void *K, const void *V, int kv_format, void *stream);

/* ATTEND.PREFIX.LOOKUP <sid> <layer> -> 1 (+HIT) if a warm slot exists, 2 (+COLD) if
 * the key is in the cold registry, 0 (+MISS) otherwise; PION_ERR_INVALID for a null
 * sid. Host-only; stamps nothing. */
int pion_prefix_lookup(const char *sid, int layer);

/* Frees the slot (sid, layer), warm or cold; layer < 0 frees every layer of sid.
 * Returns the number of keys removed (0 if none: dropping an absent key is not an
 * error), or INVALID. Waits for queued work on the device before freeing. */
int pion_prefix_drop(const char *sid, int layer);

/* Shape of a resident slot: writes H, N, D and kv_format (any pointer may be NULL).
 * For a cold key writes the shape it had and returns COLDMISS; NOT_FOUND if absent.
 * Host-only. */
int pion_prefix_info(const char *sid, int layer, int *H, int *N, int *D, int *kv_format);

/* Slot-table telemetry (the KV.PREFIX.INFO cold-tier fields of "Shared KV Cache
 * Serving": live slots, demoted entries, lifetime demotions and rehydrates), plus the
 * resident K/V bytes and the capacity in force. Host-only. */
typedef struct {
    int64_t warm_slots;      /* live (warm) slots */
    int64_t cold_slots;      /* entries in the cold registry */
    int64_t demotions;       /* lifetime WARM -> COLD transitions */
    int64_t rehydrates;      /* lifetime COLD -> WARM transitions */
    int64_t resident_bytes;  /* device K/V bytes of the warm slots */
    int64_t max_slots, max_bytes, cold_capacity;
} pion_prefix_stats_t;
int pion_prefix_stats(pion_prefix_stats_t *stats);

/* Sets the capacity (max_slots >= 1; max_bytes >= 0, 0 = no byte budget; cold_slots
 * >= 0) and demotes least recently used slots at once until it holds (then trims the
 * cold registry). INVALID for out-of-range values. */
int pion_prefix_set_capacity(int64_t max_slots, int64_t max_bytes, int64_t cold_slots);

/* ATTEND.PREFIX.QUERY <sid> <layer> <H> <D> <top_k> <Q_blob>, in its M=1 and batched-Q
 * forms ("Shared KV Cache Serving", Wire-protocol details: Q is (H, M, D), the reply is
 * H*M*D fp32 followed by an H*M fp32 LSE trailer).
 *   Q        fp16 [H_q, M, D]; row i of q-head h attends all N resident keys of
 *            kv-head head_map[h].
 *   head_map HOST int32 [H_q] or NULL (H_kv is the stored H).
 *   out      fp32 [H_q, M, D], normalized attention output.
 *   lse      fp32 [H_q, M] or NULL.
 * top_k and fa_window are not taken: the pages measure only top_k = N (dense).
 * Errors: INVALID (pointers, M < 1, H_q < 1 or > 128, D != stored D, head_map entry
 * outside [0, H_kv), H_kv not dividing H_q without a head_map), NOT_FOUND, COLDMISS,
 * HIP. Every query form below also returns COLDMISS for a cold key. */
int pion_prefix_query(const char *sid, int layer, int H_q, int D, int M,
                      const void *Q, const int32_t *head_map,
                      float *out, float *lse, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments, results and errors as
 * pion_prefix_query (the same kernels run), but every device buffer the launch plan
 * needs beyond the caller's Q, out, lse and the resident slot - the split-over-keys
 * partials and the merge's ticket counters - lives in a fixed scratch area the library
 * holds per GPU for the life of the process: 64 MiB (256 KiB of counters, the rest
 * partials). The call performs no device allocation or free. The first call on a device
 * takes that device's scratch address and clears its counters with a kernel on `stream`.
 *   Limit: a plan whose partials exceed the area returns PION_ERR_SCRATCH before any
 *   launch (pion_prefix_query serves it). The partials of a plan are at most
 *   H_q * M * D * 4 bytes times its key splits: the H_q = 24, N = 4096, M = 512, D = 128
 *   batched-Q query needs 32 MB and fits; H_q = 64, M = 512 at D = 512 (67 MB) does not.
 *   Every call on one GPU shares its scratch area and the area keeps the last call's
 *   contents: calls that overlap in time on one GPU (different streams, or host
 *   threads racing) race on it. Calls ordered on one stream are safe. */
int pion_prefix_query_noalloc(const char *sid, int layer, int H_q, int D, int M,
                              const void *Q, const int32_t *head_map,
                              float *out, float *lse, void *stream);

/* Batched form of pion_prefix_query over the layers layer0 .. layer0 + n_layers - 1 of
 * one session, computed in a single launch. Not a wire form of the pages: it issues the
 * per-layer ATTEND.PREFIX.QUERY calls of independent layers together, so the device
 * streams every layer's K/V in one pass instead of paying launch and merge latency
 * per layer. Each layer's result is exactly that of pion_prefix_query.
 *   Q    fp16 [n_layers, H_q, M, D]; out fp32 [n_layers, H_q, M, D];
 *   lse  fp32 [n_layers, H_q, M] or NULL.
 * All slots must exist (else NOT_FOUND) and share H, D and kv_format (else INVALID);
 * N may differ per layer. 1 <= n_layers <= 64. Other errors as pion_prefix_query. */
int pion_prefix_query_layers(const char *sid, int layer0, int n_layers, int H_q, int D, int M,
                             const void *Q, const int32_t *head_map, float *out, float *lse,
                             void *stream);

/* ATTEND.PREFIX.QUERY_FUSED <sid> <layer> <H_q> <D> <S_suf> <H_kv> <Q> <K_suf> <V_suf>
 * <head_map>: the caller's dense suffix attention merged with the resident prefix in
 * one call (ATTEND.* page, QUERY_FUSED row; GQA-aware).
 *   Q            fp16 [H_q, M, D] (the wire derives M from the blob; here it is explicit).
 *   K_suf, V_suf fp16 [H_kv, S_suf, D]; may be NULL when S_suf == 0.
 *   Row i of q-head h (g = head_map[h]) attends all N prefix keys of g and the suffix
 *   keys j <= S_suf - M + i of g: the suffix is causal and aligned bottom-right, so
 *   M == S_suf is the usual triangular mask and the last row sees the whole suffix.
 *   out fp32 [H_q, M, D]; lse fp32 [H_q, M] or NULL (the wire sends no trailer).
 * Errors: as pion_prefix_query, plus INVALID for H_kv != stored H, S_suf < 0,
 * M > S_suf when S_suf > 0, and null suffix pointers when S_suf > 0. */
int pion_prefix_query_fused(const char *sid, int layer, int H_q, int D, int M,
                            int S_suf, int H_kv,
                            const void *Q, const void *K_suf, const void *V_suf,
                            const int32_t *head_map, float *out, float *lse,
                            void *stream);

/* ATTEND.PREFIX.QUERY_SPARSE_AUTO <sid> <layer> <H_q> <D> <B> <K_top> <H_kv> <Q>
 * <head_map>, and with S_suf > 0 ATTEND.PREFIX.QUERY_SPARSE_AUTO_FUSED (... <S_suf> <Q>
 * <K_suf> <V_suf> <head_map>): the server picks blocks by block-mean top-K over the
 * resident K and attends only their tokens ("Shared KV Cache Serving", Stage 2,
 * sparse-mask paragraph; ATTEND.* page, QUERY_SPARSE_AUTO rows: K_mean cached per slot).
 *   Q       fp16 [H_q, 1, D] (M = 1).
 *   Blocks are tokens [b*B, min((b+1)*B, N)), nb = ceil(N/B). K_mean[g, b] is the mean
 *   of K over block b's tokens; it is computed on first use and cached in the slot per
 *   B. score[g, b] = sum over q-heads h with head_map[h] == g of q_h . K_mean[g, b].
 *   Per kv-head, the min(K_top, nb) best blocks by (score desc, block asc) are kept;
 *   q-head h attends their tokens of kv-head head_map[h], plus all S_suf suffix keys.
 *   K_suf, V_suf fp16 [H_kv, S_suf, D], NULL when S_suf == 0.
 *   out        fp32 [H_q, D]; lse fp32 [H_q] or NULL.
 *   blocks_out int32 [H_kv, K_top] or NULL: chosen blocks ascending, -1 past nb.
 * Errors: as pion_prefix_query_fused, plus INVALID for B < 1, K_top < 1,
 * K_top > 1024. */
int pion_prefix_query_sparse_auto(const char *sid, int layer, int H_q, int D,
                                  int B, int K_top, int H_kv, int S_suf,
                                  const void *Q, const void *K_suf, const void *V_suf,
                                  const int32_t *head_map, float *out, float *lse,
                                  int32_t *blocks_out, void *stream);

/* ATTEND.PREFIX.QUERY_SPARSE <sid> <layer> <H> <D> <K_sparse_max> <Q> <indices> <counts>:
 * M = 1 attention of each head over caller-supplied tokens (ATTEND.* page,
 * QUERY_SPARSE rows: per-head indices, for learned-router consumers).
 *   Q        fp16 [H, 1, D]; H is the stored H (q-head h reads kv-head h).
 *   indices  int32 [H, K_sparse_max], device memory; counts int32 [H], device memory.
 *   Head h attends tokens indices[h, j] for j < min(max(counts[h], 0), K_sparse_max);
 *   an index outside [0, N) names no token and is skipped, a repeated index is a key
 *   as many times as it is listed; a head with no key gets out 0 and lse -inf.
 *   out fp32 [H, D]; lse fp32 [H] or NULL.
 * Errors: as pion_prefix_query, plus INVALID for H != stored H, K_sparse_max < 1 or
 * > 2^24, null indices or counts; UNSUPPORTED for an mlx4g32 slot. */
int pion_prefix_query_sparse(const char *sid, int layer, int H, int D, int K_sparse_max,
                             const void *Q, const int32_t *indices, const int32_t *counts,
                             float *out, float *lse, void *stream);

/* V-store rows of one layer, as the rehydrate and fetch calls below take them: one row
 * per token, kv_dim = H * D values wide, either
 *   PION_KV_FP16     fp16 [n_rows, kv_dim] (16-byte aligned), or
 *   PION_KV_MLX4G32  the per-token record of the V-store page ("The mlx4g32 tier"):
 *                    kv_dim/8 uint32 code words, then kv_dim/32 fp16 scales, then
 *                    kv_dim/32 fp16 biases, little-endian, 5 * kv_dim / 8 bytes per
 *                    token (4-byte aligned), as pion_kv_quantize_mlx4g32 encodes a row.
 * Dequantized values are s * q + b rounded once to fp32 (an fp16 slot then rounds that
 * to fp16, nearest even). */

/* V.FETCH <sid> <layer> RANGE <start> <end> ("Shared KV Cache Serving"): the
 * concatenated dequantized fp32 values of tokens start .. end - 1.
 *   rows  device, n_rows V-store rows in format fmt (see above).
 *   out   device fp32 [end - start, kv_dim], 16-byte aligned.
 * Errors: INVALID (pointers, fmt, kv_dim <= 0 or not a multiple of 32, range outside
 * [0, n_rows], alignment), HIP. An empty range is a no-op
 * (rows and out may then be NULL). */
int pion_vstore_fetch_f32(const void *rows, int fmt, int64_t n_rows, int kv_dim,
                          int64_t start, int64_t end, float *out, void *stream);

/* KV.PREFIX.WARM, one layer ("Shared KV Cache Serving"): rehydrate the slot (sid, layer)
 * from the layer's V-store rows of K and of V (N tokens each, src_format, kv_dim = H * D),
 * transposed from the V-store layout [N, H * D] into the STORE layout [H, N, D]:
 *   kv_format FP16     the dequantized values rounded to fp16 (fp16 rows: the values);
 *   kv_format FP32     the dequantized fp32 values (the pages' own rehydrate);
 *   kv_format MLX4G32  from mlx4g32 rows: the codes, scales and biases unchanged (the same
 *                      slot a STORE of the original fp16 K/V with MLX4G32 makes); from
 *                      fp16 rows: encoded as pion_prefix_store does.
 * The slot then behaves as one made by pion_prefix_store (capacity rules, replacing a
 * live key, rehydrating a cold one). Errors: those of pion_prefix_store, and INVALID for
 * an unknown src_format or a misaligned or non-device row pointer. */
int pion_prefix_warm(const char *sid, int layer, int H, int N, int D, int src_format,
                     const void *K_rows, const void *V_rows, int kv_format, void *stream);

/* mlx4g32 encoder ("Shared KV Cache Serving", Quantized tier - mlx4g32; V-store page,
 * The mlx4g32 tier): int4 codes in groups of 32, affine, fp16 scale and bias per group,
 * the scale rounded to fp16 before codes are chosen. Per group, in fp32 with IEEE
 * rounding: mn = min, mx = max, s = fp16((mx - mn) / 15), b = fp16(mn); if s == 0 every
 * code is 0, else q = clamp(round_half_even((x - b) / s), 0, 15). Element i of a row
 * goes to word i/8 at bits 4*(i%8); the reader computes x = s*q + b.
 *   x      fp16 [rows, D], D % 32 == 0.
 *   codes  uint32 [rows, D/8]; scales, biases fp16 [rows, D/32].
 * Inputs must be finite. Errors: INVALID (pointers, rows < 0, D <= 0 or D % 32 != 0),
 * HIP. rows == 0 is a no-op. */
int pion_kv_quantize_mlx4g32(const void *x, int64_t rows, int D,
                             uint32_t *codes, void *scales, void *biases, void *stream);

/* Static description of a status code (never NULL). */
const char *pion_status_str(int status);

/* Launch-plan telemetry (not a wire form): the names, with template arguments, of the
 * kernels the calling thread's most recent call of this library enqueued, joined by
 * " + " (e.g. "prefill_kernel<128> + prefill_merge_kernel<128>"); "" if it enqueued
 * none. The string belongs to the library and stays valid until the thread's next call.
 * Host-only. */
const char *pion_prefix_last_plan(void);

/* Measurement aid (not a wire form): reads `bytes` at the device pointer buf once with
 * 16-byte non-temporal loads, one contiguous chunk per workgroup, and does nothing else -
 * the plain streaming read whose rate is the achievable ceiling the bandwidth-bound
 * kernels are compared with. sink is one
 * device uint32 the kernel may write (it does not, for realistic data). bytes must be a
 * multiple of 16 (0 is a no-op); buf 16-byte aligned. Errors: INVALID, HIP. */
int pion_bench_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* Measurement aid (not a wire form): `iters` rounds of four independent fp16 matrix
 * products (v_mfma_f32_32x32x16_f16, 32,768 flops each, the instruction of the batched-Q
 * kernels) in every wave of four 256-lane workgroups per compute unit, and nothing else -
 * the dense fp16 rate the chip sustains under full matrix load, which the batched-Q
 * kernels are compared with beside the rated peak. *flops (a host double) receives the
 * launch's flop count. sink is one device uint32 the kernel may write (it does not).
 * Errors: INVALID (iters < 1, a null or misaligned pointer), HIP. */
int pion_bench_mfma_peak(int iters, double *flops, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PION_PREFIX_H */
