/*
 * pfkv: split-KV attention for the speculative-decoding verify step over a paged
 * fp8 KV cache, native to MI355X (gfx950 / CDNA4).
 *
 * The operation (aiter PR #5190 "gfx950 assembly MTP-verify attention for
 * head_dim 256 fp8 paged KV", sections Motivation, Modifications, Kernel notes and
 * Supported; SGLang PR #37465 "gfx950 assembly attention for EAGLE verify, draft
 * extend and decode", section Modifications): for each sequence b with q_len n_b
 * query tokens (1..4) and KV length L_b, every query head attends with a softmax
 * to the first L_b positions of the paged fp8 KV cache, query i (0-based) seeing
 * positions 0 .. L_b - n_b + i (a causal mask over the last n_b positions). The
 * cache is NHD with 16-token pages (also 32 or 64 here: a page of 16 R tokens is
 * R 16-token blocks back to back; and one-token pages, where every key row is
 * gathered through its own block-table entry) and head_dim 256 (also 128 here);
 * K and V are e4m3fn bytes
 * whose real values are byte * k_descale (resp. v_descale); G = Hq / Hkv query
 * heads share each KV head, query head hq reading KV head hq / G. The pages'
 * kernel serves G = 16 and 8 (aiter PR #5190, Supported); this library also
 * serves G = 4, and G = 32 as two work-groups of 16 query heads per KV head
 * (each reads the KV head's pages, so G = 32 moves twice the K/V bytes). The
 * context of each sequence is cut into num_segments KV segments processed
 * independently; each writes partial softmax statistics to the workspace and a
 * second kernel merges them by log-sum-exp into the bf16 output.
 *
 * Threading / ownership: every buffer is owned by the caller and lives in device
 * memory of the current HIP device. The library allocates nothing per call,
 * never reads device memory from the host and never synchronizes: calls only
 * enqueue kernels on the given stream, so they are safe to capture in a HIP
 * graph. Device properties are cached per device on first use.
 */
#ifndef PFKV_H_
#define PFKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point (0 = success). */
enum pfkv_status {
  PFKV_OK = 0,
  PFKV_INVALID = 1,     /* null pointer, bad size, bad stride, too-small workspace, non-finite scale */
  PFKV_UNSUPPORTED = 2, /* valid request outside what the kernels serve: the caller should fall back */
  PFKV_DEVICE = 3,      /* a pointer is not device memory of the current device */
  PFKV_LAUNCH = 4       /* a HIP runtime error (its text is in pfkv_last_error) */
};

/* Arguments of one verify-attention call. Device pointers first, then host values. */
typedef struct pfkv_args {
  const void* q;               /* bf16 [total_q, num_q_heads, head_dim], strides below, unit last stride */
  const void* k_cache;         /* e4m3fn bytes [num_pages, page_size, num_kv_heads, head_dim], contiguous */
  const void* v_cache;         /* same layout as k_cache */
  const int32_t* block_tables; /* [num_seqs, block_table_stride]; entries in [0, num_pages) */
  const int32_t* seq_lens;     /* [num_seqs]: L_b, the KV length including the n_b query tokens */
  const int32_t* cu_seqlens_q; /* [num_seqs + 1]: prefix sums of n_b, cu[0] = 0, cu[num_seqs] = total_q */
  const float* k_descale;      /* one fp32 element */
  const float* v_descale;      /* one fp32 element */
  void* workspace;             /* >= pfkv_workspace_bytes(num_segments, total_q, num_q_heads) bytes, 16-B aligned */
  void* out;                   /* bf16 [total_q, num_q_heads, head_dim], strides below, unit last stride */
  int64_t q_stride_token;      /* elements between consecutive tokens of q */
  int64_t q_stride_head;       /* elements between consecutive heads of q */
  int64_t out_stride_token;
  int64_t out_stride_head;
  int64_t block_table_stride;  /* elements between rows of block_tables (>= max_pages_per_seq) */
  uint64_t workspace_size;     /* bytes available at workspace */
  int32_t num_seqs;            /* N >= 1 */
  int32_t total_q;             /* T = cu_seqlens_q[N], 1 <= T <= max_q_len N */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv, Hq % Hkv == 0 */
  int32_t head_dim;            /* 256 (the pages' kernel) or 128; q, out and both caches share it */
  int32_t page_size;           /* 16 (the pages' kernel), 32, 64 or 1 (one table entry per token) */
  int32_t num_pages;           /* pages in k_cache / v_cache */
  int32_t max_pages_per_seq;   /* columns of block_tables that may be read */
  int32_t num_segments;        /* S in [1, 64] */
  float softmax_scale;         /* multiplies q . k (after descale); finite and > 0 */
  int32_t precision;           /* PFKV_PRECISION_* below */
  float* lse;                  /* optional, NULL = not written: fp32 [num_q_heads, total_q], element (h, t)
                                  at lse[h * total_q + t], 4-B aligned; see below */
  const float* sinks;          /* optional, NULL = none: fp32 [num_q_heads] sink logits, 4-B aligned */
  int32_t window_keys;         /* > 0: a query sees only its window_keys most recent keys (itself included);
                                  <= 0 (the zero-initialised default): all */
  float softcap;               /* > 0: every score s becomes softcap * tanh(s / softcap); 0: off */
  int32_t max_q_len;           /* bound on every n_b: 0 (the zero-initialised default) = 4, the pages'
                                  bound; up to 8 (longer drafts); rows of tokens past it are not written */
  int32_t balance_segments;    /* 0 (default): every sequence is cut into num_segments segments. 1: segments
                                  in proportion to each sequence's pages (see below); num_segments (2..128)
                                  is then the cap per sequence and num_seqs must be <= 1024 */
  void* merge_sync;            /* optional, NULL (default) = off: sync words of the in-launch merge (below),
                                  256-B aligned, zero before the first call that uses them */
  uint64_t merge_sync_size;    /* bytes at merge_sync */
  int32_t merge_wait_us;       /* in-launch merge: how long a work-group waits for the rest of its group;
                                  0 (default) = 50 us; < 0 = not at all (each work-group that is not the last
                                  of its group hands its rows to the last: slower, same bits) */
} pfkv_args;

/*
 * In-launch merge (opt-in). The segment reduce is a second launch, which costs
 * about 5 us after a 55 us main kernel and more, relative to the call, on
 * short contexts with many segments; aiter PR #5190 (Microbenchmark, the S = 64
 * row of the bandwidth sweep) and SGLang PR #37465 (Draft shapes, decode) time
 * such calls. With merge_sync set, pfkv_verify_attn_fwd (and the
 * allocation-free entry point) run the merge inside the main launch when the
 * call allows it: 16-bit arithmetic, head_dim 256, page_size >= 16, no balanced
 * segments, num_segments >= 2, a grid of at most one work-group per CU and o
 * partials under 2 GiB. Other calls run the two launches and leave merge_sync
 * untouched. The result is bit for bit that of the two launches. Measured, it
 * pays at decode (one query token, 16 query heads per work-group, 16
 * segments: 0.8 to 1.2 us of 56 at 16 x 35000) and costs elsewhere: about 2%
 * on 4-token drafts at up to 16 segments (the merge's synchronization and
 * loads take as long as the launch boundary and the reduce), 4 to 16% above
 * 16 segments, where the two launches read row-major partials.
 * The work-groups of a (sequence, head group) count their arrivals in
 * merge_sync; once all have written their partials each merges a share of the
 * group's rows with the reduce's arithmetic. A work-group waits at most
 * merge_wait_us for the others (so none waits on one that cannot start) and
 * otherwise hands its share to the last arrival. The words must be zero
 * before the first call that uses them; every call leaves them ready for the
 * next. Calls that use the same words concurrently race: give each stream its
 * own. Size: at least pfkv_merge_sync_bytes(num_seqs, num_q_heads) bytes.
 */
uint64_t pfkv_merge_sync_bytes(int num_seqs, int num_q_heads);

/*
 * Balanced segments (balance_segments = 1), for batches whose contexts differ
 * widely (draft extend and decode): the launch has about one work-group per
 * CU, `slots` = max(num_seqs, CUs / work-groups per (sequence, segment)) of
 * them, and sequence b, whose segments split span_b pages, gets
 * min(num_segments, 1 + floor((slots - num_seqs) span_b / sum of spans))
 * segments. The schedule is computed on the device from seq_lens (so the call
 * stays capturable); a sequence's result depends on the other sequences'
 * lengths through it, not on their queries.
 */

/*
 * Options that the pages name only as features their gates leave out (SGLang
 * PR #37465, Modifications: no sliding window, soft-cap or sinks; aiter PR
 * #7375, Changes: windows, sinks, soft-cap), in their common reading. With a
 * score s_j = softmax_scale * <q, k_j> (K descaled):
 *  - window_keys = W + 1 > 0: query i of a sequence (position L - n + i) sees
 *    keys L - n + i - W .. L - n + i, i.e. a left window of W positions (the
 *    convention that aiter PR #7375, Changes, applies, where a negative left
 *    window is unlimited; here 0 keeps zero-initialised arguments unlimited).
 *    The segments then partition only the pages some query can see.
 *  - softcap c > 0: s_j -> c tanh(s_j / c) before the softmax.
 *  - sinks: out = sum_j e^(s_j) v_j / (sum_j e^(s_j) + e^(sink_h)) and the sink
 *    adds e^(sink_h) to the lse sum: a probability mass that carries no value.
 */

/*
 * Log-sum-exp output (aiter PR #7375, Summary and Behavior and intent: an
 * optional LSE in the varlen layout (heads, total tokens), computed from the
 * same rounded softmax weights that normalise the output, so that output and
 * LSE stay consistent for a later log-sum-exp merge of partial attentions).
 * lse[h][t] = ln sum_j exp(softmax_scale * <q_t,h , k_j>) over the keys j the
 * row may see (K descaled), where each exp is the probability the kernel
 * weighted V with: p_j = 2^(c s_j - m) rounded as P is rounded (fp16, or e4m3
 * for the fp8 P variants), so lse = ln 2 * (m + log2 sum_j p_j). It differs
 * from the exact value by the relative rounding of P (at most 2^-11 with fp16
 * P, i.e. 5e-4 in lse). A row with no visible key gets -inf (aiter PR #7375,
 * review thread: non-finite reference rows are -inf). Written by the segment
 * reduce, or by the main kernel when num_segments == 1.
 */

/*
 * Arithmetic of the main kernel.
 * PFKV_PRECISION_16BIT (0, the default): Q in bf16 against K converted exactly
 *   to bf16; P rounded once to fp16 against V converted exactly to fp16; fp32
 *   accumulation.
 * PFKV_PRECISION_FP8_P (1): scores as in the default; P rounded to e4m3 and
 *   P V on the fp8 MFMA against the cached e4m3 V bytes.
 * PFKV_PRECISION_FP8 (2): the pages' precision class (aiter PR #5190, Kernel
 *   notes and Accuracy): each query row quantised to e4m3 with scale amax / 448
 *   and both contractions on the fp8 MFMA.
 * With e4m3 P, probabilities below 2^-10 of a row's reference maximum flush to
 * zero (the underflow the aiter PR #7375 review thread works through). With
 * e4m3 Q, rows that see only a handful of keys can flip close maxima (errors of
 * 0.5 sigma and more measured with 8 visible keys); the fp8 variants are meant
 * for long contexts.
 */
enum pfkv_precision { PFKV_PRECISION_16BIT = 0, PFKV_PRECISION_FP8_P = 1, PFKV_PRECISION_FP8 = 2 };

/*
 * Pure host-side validation; reads no device memory and needs no GPU. It is the
 * argument check of the launcher that aiter PR #5190 describes (Modifications:
 * the C++ launcher validates its arguments before the two launches; Supported:
 * what is outside the supported set is rejected by a check).
 * arch: the device's gcnArchName (e.g. "gfx950:sramecc+:xnack-"); anything not
 * starting with "gfx950" is PFKV_UNSUPPORTED. num_cus: compute units (> 0).
 * Returns a pfkv_status; on failure pfkv_last_error() says which check failed.
 * Device-side preconditions that are NOT checked here (they would need a device
 * read): 0 <= n_b <= max_q_len (4 when max_q_len is 0), n_b <= L_b <=
 * page_size * max_pages_per_seq, and block table entries in [0, num_pages).
 * The kernels clamp each of them so that no access leaves its buffer; results
 * for inputs that break them are unspecified.
 */
int pfkv_check_args(const pfkv_args* args, const char* arch, int num_cus);

/*
 * Enqueue the verify-attention call on `stream` (a hipStream_t; NULL = the null
 * stream): the split-KV main kernel on a grid of num_segments x num_seqs x
 * (num_kv_heads * kv_split * q_split) work-groups, kv_split = 2 when G = 32 (two
 * work-groups of 16 query heads per KV head) and q_split = 2 when 16 query heads
 * per work-group meet max_q_len > 4 (two blocks of at most 4 query tokens),
 * each 1 otherwise; then the segment reduce. With num_segments == 1
 * the main kernel writes out itself and no reduce is enqueued (the workspace is
 * still validated but not touched). Validates with
 * pfkv_check_args against the current device first and checks that the device
 * pointers belong to it (each thread remembers the last 32 pointers it found to
 * be device memory of a device and does not query them again, so a loop that
 * passes the same buffers makes no queries). Aliasing between out and any
 * input is not allowed.
 * Concurrent calls that share a workspace race; give each stream its own.
 */
int pfkv_verify_attn_fwd(const pfkv_args* args, void* stream);

/*
 * Debug mode: on (PFKV_DEBUG=1 in the environment at the first call, or
 * pfkv_set_debug(1)), pfkv_verify_attn_fwd and pfkv_splitkv_main first run a
 * checking kernel over the device-side preconditions above (cu_seqlens_q
 * monotone from 0 to total_q, 0 <= n_b <= max_q_len, n_b <= L_b <= page_size *
 * max_pages_per_seq, used block-table entries in [0, num_pages)) and return
 * PFKV_INVALID, naming the first offending sequence, without launching the
 * attention kernels. Debug mode synchronizes the stream and allocates a 16-byte
 * status buffer per device once: it is not for graph capture. Returns the
 * previous setting.
 */
int pfkv_set_debug(int on);

/*
 * pfkv_verify_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same validation, kernels and results, but the per-segment partials go to a
 * device array the library holds (PFKV_NOALLOC_SCRATCH_BYTES bytes on each GPU it
 * runs on, until the process ends) instead of args->workspace, which is ignored
 * (it may be NULL, workspace_size 0). A call whose partials need more
 * (pfkv_workspace_bytes(num_segments, total_q, num_q_heads) > the limit) returns
 * PFKV_INVALID. It calls no allocating routine and does not run the debug check.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race; serialize them.
 */
#define PFKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int pfkv_verify_attn_fwd_noalloc(const pfkv_args* args, void* stream);

/*
 * The two stages of pfkv_verify_attn_fwd, exposed separately (same arguments,
 * same validation) so that a caller can place or time them individually:
 * pfkv_splitkv_main enqueues only the split-KV main kernel, which writes the
 * per-segment partials to the workspace; pfkv_segment_reduce enqueues only the
 * reduce that turns the workspace into out. Running them in this order on one
 * stream is exactly pfkv_verify_attn_fwd. With num_segments == 1,
 * pfkv_splitkv_main writes out directly and pfkv_segment_reduce enqueues nothing.
 */
int pfkv_splitkv_main(const pfkv_args* args, void* stream);
int pfkv_segment_reduce(const pfkv_args* args, void* stream);

/*
 * Segment-count heuristic (aiter PR #5190, Modifications: a helper that picks
 * the number of segments; Kernel notes: one work-group per CU):
 * clamp(num_cus / (num_seqs * num_kv_heads), 1, 64). Pure; returns 0 for
 * non-positive inputs. A call runs num_seqs * num_kv_heads * kv_split * q_split
 * work-groups per segment (pfkv_verify_attn_fwd); passing num_kv_heads *
 * kv_split * q_split as num_kv_heads keeps one work-group per CU for 32 query
 * heads per KV head or more than 4 query tokens with 16 query heads per
 * work-group.
 */
int pfkv_num_segments(int num_cus, int num_seqs, int num_kv_heads);

/*
 * Workspace bytes for S segments (aiter PR #5190, Modifications: the Python
 * entry point allocates the split-KV workspaces the launcher writes and the
 * reduce reads): S * total_q * num_q_heads * 520. 0 for bad sizes. Layout (after the main kernel): fp16 o[S][total_q][num_q_heads][256],
 * the segment's softmax-weighted mean of V (without v_descale, 0 for a segment
 * with no visible key; at head_dim 128 the first 128 of each row), then fp32 (m, l)[S][total_q][num_q_heads], m the
 * segment's reference max of the scores in log2 units (-inf when empty) and
 * l the sum of 2^(score - m) over its keys. Above 16 segments in the 16-bit
 * mode at head_dim 256 with pages of 16 tokens or more, both arrays are
 * row-major instead, o[total_q][num_q_heads][S][256] and (m, l)[total_q]
 * [num_q_heads][S], so that a row's partials are contiguous for the reduce
 * (pfkv_partials_row_major).
 */
uint64_t pfkv_workspace_bytes(int num_segments, int total_q, int num_q_heads);

/*
 * 1 when a call with these arguments leaves its workspace partials row-major
 * (layout above), 0 when segment-major; the same test the call itself makes,
 * for callers that read the partials (for instance to merge them with those of
 * another chunk of keys, the split-softmax merge of aiter PR #5190,
 * Modifications). precision is a PFKV_PRECISION_* value. Pure: no device is
 * touched and any values are accepted (0 for the ones a call would refuse).
 */
int pfkv_partials_row_major(int precision, int head_dim, int page_size, int num_segments);

/*
 * Text of the most recent failure on this host thread ("" if none), naming the
 * check that failed (aiter PR #5190, Supported: unsupported inputs are rejected
 * by a check rather than run). Valid until the next call on the thread.
 */
const char* pfkv_last_error(void);

/*
 * Properties of HIP device `device` as the library caches them: its gcnArchName
 * (copied NUL-terminated into arch, at most arch_len bytes) and CU count.
 */
int pfkv_device_info(int device, char* arch, int arch_len, int* num_cus);

/*
 * Streaming-read microbenchmark kernels (aiter PR #5190, Microbenchmark: a
 * streaming-read microbenchmark that bounds the achievable read rate). Reads
 * `bytes` bytes of `buf` once, as 4 KiB blocks, with one work-group of 8 waves
 * per CU:
 *   variant 0: blocks in address order, 16-byte vector loads into registers;
 *   variant 1: blocks in address order through LDS with global_load_lds_dwordx4
 *              (each block read back from LDS);
 *   variant 2: as 1, visiting blocks in the order given by page_order
 *              (num_pages int32 block indices in [0, bytes / 4096); out-of-range
 *              entries are clamped);
 *   variant 3: as 0, in the order given by page_order.
 * Every 32-bit word read is XORed into the 4-byte device word `sink` (atomic
 * XOR, not cleared here): with sink zeroed first and page_order a permutation
 * of all blocks, sink ends as the XOR of the whole buffer, which proves that
 * every byte was read. bytes must be a positive multiple of 4096, buf 16-byte
 * aligned, sink 4-byte aligned; all pointers device memory of the current
 * device. Enqueues one kernel on `stream`; returns a pfkv_status.
 */
int pfkv_stream_read(const void* buf, uint64_t bytes, int variant, const int32_t* page_order,
                     int64_t num_pages, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PFKV_H_ */
