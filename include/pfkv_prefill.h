/*
 * pfkv prefill: fp8 varlen prefill attention, the second workload of this
 * library, native to MI355X (gfx950 / CDNA4). Status codes and
 * pfkv_last_error() are those of pfkv.h.
 *
 * The operation (aiter PR #7375 "gfx1250 fp8 varlen FMHA", sections Summary and
 * Changes): for each sequence b of a packed varlen (THD) batch, with Lq_b query
 * rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and Lk_b key/value rows
 * cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1, every query head hq attends with a
 * softmax over scores softmax_scale * <q, k> to the sequence's keys of KV head
 * hq / (Hq / Hkv). Q, K and V are e4m3fn bytes whose real values are
 * byte * q_descale (k_descale, v_descale), the descales being single fp32
 * values read from device memory. The qk head dim is 192 and the v head dim
 * 128. With causal != 0 the mask is aligned to the bottom right: query i sees
 * keys 0 .. Lk_b - Lq_b + i. A query that sees no key gets 0 (and lse -inf).
 *
 * Arithmetic: S = Q K^T on the e4m3 MFMA with fp32 accumulation (exact
 * products); P in e4m3 with a power-of-two scale per 32 keys of a row (the
 * MFMA's E8M0 block scales), so that small probabilities keep 3 mantissa bits
 * rather than flushing to zero; O = P V on the same MFMA; the row sum l and the
 * lse come from the same rounded weights as O.
 *
 * Ownership and threading as in pfkv.h: caller-owned device buffers on the
 * current device, no allocation, no host reads of device data, no
 * synchronization; one kernel is enqueued on the given stream.
 */
#ifndef PFKV_PREFILL_H_
#define PFKV_PREFILL_H_

#include <stdint.h>

#include "pfkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pfkv_prefill_args {
  const void* q;               /* e4m3fn bytes [total_q, Hq, 192] */
  const void* k;               /* e4m3fn bytes [total_k, Hkv, 192] */
  const void* v;               /* e4m3fn bytes [total_k, Hkv, 128] */
  void* out;                   /* bf16 [total_q, Hq, 128] */
  float* lse;                  /* optional (NULL = not written): fp32 [Hq, total_q], natural log */
  const int32_t* cu_seqlens_q; /* [num_seqs + 1] device, 0 .. total_q, nondecreasing */
  const int32_t* cu_seqlens_k; /* [num_seqs + 1] device, 0 .. total_k, nondecreasing */
  const float* q_descale;      /* one fp32 element each, device */
  const float* k_descale;
  const float* v_descale;
  int64_t q_stride_token, q_stride_head;     /* bytes; positive multiples of 16 */
  int64_t k_stride_token, k_stride_head;     /* bytes; positive multiples of 16 */
  int64_t v_stride_token, v_stride_head;     /* bytes; positive multiples of 16 */
  int64_t out_stride_token, out_stride_head; /* elements; positive multiples of 4 */
  int32_t num_seqs;            /* 1 .. 65535 */
  int32_t total_q;             /* rows of q and out (>= 1) */
  int32_t total_k;             /* rows of k and v (>= 0) */
  int32_t num_q_heads;         /* 1 .. 65535, a multiple of num_kv_heads */
  int32_t num_kv_heads;        /* >= 1 */
  int32_t head_dim_qk;         /* must be 192 */
  int32_t head_dim_v;          /* must be 128 */
  int32_t max_seqlen_q;        /* bound on every Lq_b, >= 1; ceil(max_seqlen_q / 256) * num_q_heads < 2^31 */
  float softmax_scale;         /* finite, > 0 (the usual choice is 1 / sqrt(192)) */
  int32_t causal;              /* 0: full attention; else bottom-right causal */
} pfkv_prefill_args;

/*
 * Pure argument validation (no GPU calls), as pfkv_check_args. Returns
 * PFKV_INVALID for a malformed request (NULL pointer, bad count, stride or
 * alignment), PFKV_UNSUPPORTED for a valid one the kernel does not serve (head
 * dims other than 192 / 128, arch not gfx950), else PFKV_OK.
 */
int pfkv_prefill_check_args(const pfkv_prefill_args* a, const char* arch, int num_cus);

/*
 * Validates (pfkv_prefill_check_args with the cached device arch, then that
 * every pointer is device memory of the current device: PFKV_DEVICE otherwise)
 * and enqueues the prefill kernel on `stream` (a hipStream_t; NULL = the null
 * stream). Device-side preconditions, not checked on the host: cu_seqlens as
 * documented above and Lq_b <= max_seqlen_q; the kernel clamps every sequence
 * into the buffers, so a violation gives wrong values, never an access outside
 * them.
 */
int pfkv_prefill_fwd(const pfkv_prefill_args* a, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PFKV_PREFILL_H_ */
