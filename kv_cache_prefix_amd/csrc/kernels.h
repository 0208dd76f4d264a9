// Internal launch interface between the C ABI (pion_prefix.cpp) and the HIP kernels.
// Not installed; the public interface is include/pion_prefix.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pion {

// Records the name (printf-style, with its template arguments) of a kernel a launch
// function enqueues; the C ABI keeps the names of the current call's launches for
// pion_prefix_last_plan. Defined in pion_prefix.cpp; host only.
void note_launch(const char *fmt, ...) __attribute__((format(printf, 1, 2)));

constexpr int kMaxHeads = 128;     // H_q limit (row-group table size)
constexpr int kRowsPerGroup = 8;   // q-heads sharing one kv-head read per workgroup

// Groups of up to kRowsPerGroup q-heads that read the same kv-head. A workgroup of the
// partial-attention kernel serves one group at one query index, so the K/V bytes it
// streams are shared by every q-head of the group (GQA). Group i: gc[i] = kv-head |
// rows << 8; heads[i] = its q-heads, row r in byte r of the 64-bit word. Whole words, so
// a kernel reads its group with two scalar loads at entry.
struct RowGroups {
  int n;
  uint32_t gc[kMaxHeads];
  uint64_t heads[kMaxHeads];
};
static_assert(kRowsPerGroup <= 8, "a group's q-heads are the bytes of one 64-bit word");

constexpr int kMaxBatch = 64;     // problems (layers) per launch

// Head dims served: the pages' full set. Every one is a multiple of 32 (one mlx4g32
// group), so a row is whole 16-byte pieces of fp16 and whole groups of codes.
__host__ __device__ constexpr bool head_dim_supported(int D) {
  return D == 32 || D == 64 || D == 96 || D == 128 || D == 160 || D == 192 || D == 256 ||
         D == 512;
}
__host__ __device__ constexpr int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p *= 2;
  return p;
}
// Lanes that read one fp16 key row in the VALU kernels: one per 16 bytes, rounded up to
// a power of two (lanes past D/8 hold no dims).
__host__ __device__ constexpr int fp16_row_lanes(int D) { return pow2_ceil(D / 8); }
constexpr int kGatherChunk = 2048;  // token-list positions per span

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Byte offsets of the arrays inside one slot allocation; host (store) and device
// (query) both derive pointers from this. fmt 0 fp16 / fmt 2 fp32: K, V [H, N, D]. fmt 1
// mlx4g32: K codes
// [H, N, D/8] u32, K scale/bias pairs [H, N, D/32] u32 (fp16 scale in the low half,
// fp16 bias in the high half), then the same two for V. A lane that owns one group of
// one token reads its 16 code bytes and its 4-byte pair with two loads.
struct SlotLayout {
  size_t off[4];
  size_t bytes;
};

__host__ __device__ inline SlotLayout slot_layout(int fmt, int H, int N, int D) {
  SlotLayout L;
  const size_t elems = (size_t)H * N * D;
  if (fmt != 1) {
    const size_t b = (elems * (fmt == 2 ? 4 : 2) + 255) & ~(size_t)255;
    L.off[0] = 0;
    L.off[1] = b;
    L.off[2] = L.off[3] = 0;
    L.bytes = 2 * b;
  } else {
    const size_t cb = (elems / 2 + 255) & ~(size_t)255;   // codes: 4 bits per element
    const size_t sb = (elems / 8 + 255) & ~(size_t)255;   // pairs: 4 bytes per 32 elements
    L.off[0] = 0;
    L.off[1] = cb;
    L.off[2] = cb + sb;
    L.off[3] = 2 * cb + sb;
    L.bytes = 2 * cb + 2 * sb;
  }
  return L;
}

// One resident prefix as the kernels see it.
struct KVView {
  int fmt;              // 0 fp16, 1 mlx4g32, 2 fp32
  int H, N, D;
  const void *K, *V;                     // fp16 or fp32 [H, N, D]
  const uint32_t *Kc, *Vc;               // mlx4g32 codes [H, N, D/8]
  const uint32_t *Ksb, *Vsb;             // mlx4g32 (scale | bias << 16) [H, N, D/32]
};

__host__ __device__ inline KVView make_view(const void *base, int fmt, int H, int N, int D) {
  const SlotLayout L = slot_layout(fmt, H, N, D);
  const char *b = (const char *)base;
  KVView v;
  v.fmt = fmt;
  v.H = H;
  v.N = N;
  v.D = D;
  v.K = v.V = nullptr;
  v.Kc = v.Vc = nullptr;
  v.Ksb = v.Vsb = nullptr;
  if (fmt != 1) {
    v.K = b + L.off[0];
    v.V = b + L.off[1];
  } else {
    v.Kc = (const uint32_t *)(b + L.off[0]);
    v.Ksb = (const uint32_t *)(b + L.off[1]);
    v.Vc = (const uint32_t *)(b + L.off[2]);
    v.Vsb = (const uint32_t *)(b + L.off[3]);
  }
  return v;
}

// Split-over-keys attention for up to kMaxBatch independent problems (resident slots
// of identical H, D and format, e.g. the layers of one session) in one launch.
// Workgroup (x, y, z): z = problem, y = head group * M + query index, x = key span.
// A problem's keys are segments: [0, pre_splits) cover the prefix (dense chunks of
// pre_chunk tokens, or with `blocks` one selected block each), then suf_splits chunks
// of suf_chunk suffix tokens clipped to the causal limit. Span x covers segments
// [x * seg_per_span, (x + 1) * seg_per_span) (seg_per_span is 1 for an mlx4g32 slot,
// whose prefix and suffix run in separate launches); a problem with a single span
// writes out and lse directly.
// Partials (acc unnormalized against m; m and l in log2 units) of problem z go to
// part_acc + z*part_stride as [M][H_q][S_max][D] and part_m / part_l + z*ml_stride as
// [M][H_q][S_max] (query index outermost, so the rows of one query index lie within
// H_q*S_max*D*4 bytes); the last workgroup of each (z, y) (ticket on
// counters[z*y_groups+y], which start at zero and are left at zero) merges them into
// out and lse.
struct PartialParams {
  int H_q, M, D, H_kv, fmt;
  int esz;                // bytes per element of Q and the suffix: 4 for an fp32 slot, else 2
  int waves;              // waves per workgroup of the fp16 kernel: 4, or 8 (rows <= 4)
  float qscale;           // log2(e) / sqrt(D)
  int n_prob;
  const void *Q;          // fp16 (fp32 for an fp32 slot) [n_prob][H_q, M, D]
  size_t q_stride;
  float *out;             // [n_prob][H_q, M, D]
  size_t out_stride;
  float *lse;             // [n_prob][H_q, M] or null
  size_t lse_stride;
  int pre_chunk;
  const int32_t *blocks;  // [H_kv, K_top] or null (single problem only)
  int K_top, B, n_sel;
  // caller-supplied token lists (single problem, one q-head per kv-head): q-head h
  // attends tokens gidx[h, j] for j < min(max(gcount[h], 0), gmax); indices outside
  // [0, N) are skipped. The prefix segments then chunk the list positions [0, gmax).
  const int32_t *gidx, *gcount;  // [H, gmax], [H] or null
  int gmax;
  const void *Ksuf, *Vsuf;  // fp16 (fp32) [H_kv, S_suf, D] (single problem only)
  int S_suf, suf_chunk, suf_splits;
  int seg_per_span;       // segments per span (>= 1)
  int S_max;              // span stride of the partial layout
  int x_begin;            // span index of this launch's blockIdx.x == 0
  float *part_acc, *part_m, *part_l;
  size_t part_stride, ml_stride;
  int *counters;
  int y_groups;
  // (the scalars and pointers above come first: the few cache lines every workgroup
  // reads at entry; then the per-problem and per-group tables, of which it reads one
  // entry each)
  const void *kv_base[kMaxBatch];
  int N[kMaxBatch];
  // per problem: its prefix segments | its spans (S_total) << 16, both below 2^16;
  // computed by the host, so a workgroup knows its problem's shape from two loads
  uint32_t spans[kMaxBatch];
  RowGroups rg;
};

// q-head -> kv-head, for kernels that need the whole map.
struct HeadMap {
  int H_q;
  uint8_t m[kMaxHeads];
};

// Launch spans [x_begin, x_begin + x_count) of every problem. launch_partial runs the
// fp16 kernel (prefix spans of an fp16 slot, suffix spans; it skips prefix spans of an
// mlx4g32 slot); launch_partial_mlx4 the mlx4g32-prefix kernel (it skips suffix spans,
// and takes rows_per_group <= kMlx4Rows).
constexpr int kMlx4Rows = 4;
hipError_t launch_partial(const PartialParams &p, int rows_per_group, int x_count, hipStream_t s);
hipError_t launch_partial_mlx4(const PartialParams &p, int rows_per_group, int x_count,
                               hipStream_t s);
// The same spans of an mlx4g32 prefix at D = 128 on fp16 MFMA (rows_per_group <= 4).
hipError_t launch_mlx4_mfma(const PartialParams &p, int rows_per_group, int x_count,
                            hipStream_t s);
// Batched-Q attention on fp16 MFMA over a resident fp16 prefix plus an optional fp16
// causal suffix (bottom-right aligned). A workgroup serves (tile, split): tile = (q-head,
// block of 128 query rows), split = a range of split_keys tokens of the concatenated key
// index [0, N + S_suf). With n_splits > 1 the splits store partials (each split's
// normalized output in fp16: [tile][n_splits][128 * D] in the kernel's register layout;
// its log-sum-exp in log2 units: [H_q*M][n_splits]) and prefill_merge_kernel, launched
// next on the same stream, merges them into out and lse.
// The 1-D grid is ordered so that the workgroups of one kv-head share an XCD:
// order[] lists the q-heads grouped by kv-head.
struct PrefillParams {
  const uint16_t *Q;              // fp16 [H_q, M, D]
  const uint16_t *K, *V;          // fp16 [H_kv, N, D]
  const uint16_t *Ksuf, *Vsuf;    // fp16 [H_kv, S_suf, D] or null
  int H_q, M, D, H_kv, N, S_suf;
  float qscale;                   // log2(e) / sqrt(D)
  int n_iblk;                     // ceil(M / 128)
  int n_splits, split_keys;       // split_keys a multiple of 32
  float *out, *lse;
  uint16_t *part_acc;             // split partials (n_splits > 1): fp16 normalized outputs
  float *part_lse;                // and per [row][split] log-sum-exp (log2 units)
  HeadMap hm;
  uint8_t order[kMaxHeads];       // q-heads sorted by kv-head
};

hipError_t launch_prefill(const PrefillParams &p, hipStream_t s);

// V-store rows of one layer (kv = H * D values per token): fmt 0 = fp16 [N, kv], fmt 1 =
// mlx4g32 records of 5 * kv / 8 bytes. Fetch: fp32 [count, kv] of tokens start ..
// start + count - 1. Relayout into a slot: fp16 [H, N, D] (dequantized and rounded for
// fmt 1), fp32 [H, N, D] (dequantized), or, from fmt 1, mlx4g32 codes [H, N, D/8] and
// (scale | bias << 16) pairs [H, N, D/32].
hipError_t launch_vstore_fetch(const void *rows, int fmt, int kv, int64_t start, int64_t count,
                               float *out, hipStream_t s);
hipError_t launch_rows_to_fp16_slot(const void *rows, int fmt, int64_t N, int H, int D,
                                    uint16_t *dst, hipStream_t s);
hipError_t launch_rows_to_fp32_slot(const void *rows, int fmt, int64_t N, int H, int D,
                                    float *dst, hipStream_t s);
hipError_t launch_rows_to_mlx4_slot(const void *rows, int64_t N, int H, int D, uint32_t *codes,
                                    uint32_t *pairs, hipStream_t s);

// Read `bytes` (a multiple of 16) at buf once with 16-byte non-temporal loads and
// nothing else (the streaming-read ceiling); sink receives at most one word.
hipError_t launch_stream_read(const void *buf, int64_t bytes, uint32_t *sink, hipStream_t s);
// iters rounds of four independent fp16 MFMA products in every wave of four 256-lane
// workgroups per CU (the sustained MFMA ceiling); *flops (host) gets the launch's flops.
hipError_t launch_mfma_peak(int iters, double *flops, uint32_t *sink, hipStream_t s);

// Ticket counters of a workspace: one per workgroup row of a split launch.
constexpr int kMaxCounters = 65536;

// The fixed scratch of pion_prefix_query_noalloc: kMaxCounters ticket counters, then the
// split partials. noalloc_scratch returns this device's copy (its address taken once per
// device, the counters cleared on `s` at that first call).
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
constexpr size_t kNoallocCounterBytes = (size_t)kMaxCounters * 4;
hipError_t noalloc_scratch(hipStream_t s, void **ptr);

// Zero the ticket counters of a fresh workspace.
hipError_t launch_zero_counters(int *counters, int n, hipStream_t s);

// Encode rows x [rows, D] (fp16) as mlx4g32: codes [rows, D/8] u32; the scale and bias
// of group i go to scales[i * sb_stride] and biases[i * sb_stride] (sb_stride 1 for
// separate arrays, 2 for interleaved (scale, bias) pairs).
hipError_t launch_quantize_mlx4g32(const uint16_t *x, int64_t rows, int D, uint32_t *codes,
                                   uint16_t *scales, uint16_t *biases, int sb_stride,
                                   hipStream_t s);

}  // namespace pion
