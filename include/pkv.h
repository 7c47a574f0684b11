/*
 * pkv.h -- C ABI of libpkv: one decode step of paged-KV attention on an
 * AMD MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * A decode step gives every running request exactly one new token: its K/V
 * row is appended to the request's cache and its query attends over the
 * request's whole K/V history ("Disaggregated LLM Serving：从 PD 分离到
 * Attention 卸载", section 1, and section 2.1 on one query token per decode
 * request).  The history lives in fixed-size physical blocks of a shared pool;
 * each request owns a page table that maps its logical blocks to physical ones,
 * in any order ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section
 * 2.2).  Block allocation and all per-request metadata are prepared by the
 * caller before the step, off the critical path, and the query/key/value of a
 * step may arrive as one packed buffer ("Injecting Adrenaline into LLM Serving"
 * review, section 3.2.1: metadata moved off the critical path, q/k/v sent as
 * one aggregated transfer).  The attention is standard scaled-dot-product
 * softmax attention; query head h reads KV head h / (H_q / H_kv).
 *
 * Memory layout (all device memory is owned by the caller)
 * ------------------------------------------------------
 *   k_pool, v_pool : [n_blocks][H_kv][block_size][D]   storage dtype
 *   block_tables   : [B][bt_stride] int32; entry j of row b is the physical
 *                    block holding tokens j*block_size .. j*block_size+block_size-1
 *   context_lens   : [B] int32, tokens attention reads for request b
 *   positions      : [B] int32, slot index of the token being appended
 *   q              : [B][H_q][D] storage dtype; rows (requests) q_row_stride
 *                    elements apart, heads D elements apart
 *   k_new, v_new   : [B][H_kv][D] storage dtype; rows new_row_stride apart
 *                    (so q, k_new, v_new may be views into one packed qkv row)
 *   out            : [B][H_q][D] float32, contiguous
 * All pointers must be 16-byte aligned and all row strides multiples of 8
 * bytes' worth of elements (16 bytes for D >= 64); the library checks this.
 *
 * Supported set
 * -------------
 *   dtype      : PKV_F32, PKV_F16, PKV_BF16 (out is always float32)
 *   D          : 64 or 128
 *   block_size : 16
 *   H_q % H_kv == 0; G = H_q / H_kv <= 16 on the grouped (matrix-core) path
 *   (f16/bf16); f32 with G > 1 runs per query head.
 *
 * Calling convention
 * ------------------
 * Every entry point validates its host-side arguments first and returns a
 * negative pkv_status without launching anything if they are wrong; the
 * detail is in pkv_last_error() (thread-local).  On success the work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and the call
 * returns without synchronising; results are valid once the stream reaches
 * that point.  No entry point allocates device memory, and calls on different
 * streams may overlap freely as long as their outputs do not alias.
 *
 * Device-side metadata (block ids, lengths, positions) is read by the kernels
 * and checked there: a block id outside [0, n_blocks) or a length outside
 * [0, max_context_len] never causes an out-of-bounds access.  Attention writes
 * a NaN output row for such a request; kv_append skips such a request.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PKV_F32 = 0,
    PKV_F16 = 1,
    PKV_BF16 = 2
} pkv_dtype;

typedef enum {
    PKV_OK = 0,
    PKV_ERR_NULL = -1,          /* a required pointer is NULL                           */
    PKV_ERR_INVALID_ARG = -2,   /* sizes, strides or alignment are inconsistent          */
    PKV_ERR_UNSUPPORTED = -3,   /* valid, but outside the supported set above            */
    PKV_ERR_WORKSPACE = -4,     /* workspace missing or smaller than required            */
    PKV_ERR_HIP = -5            /* the HIP runtime reported an error when launching      */
} pkv_status;

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Human-readable name of a pkv_status value. */
const char* pkv_status_string(int status);

/* Detail of the last non-OK return on this thread ("" if none). */
const char* pkv_last_error(void);

/* Launch geometry of the last successful attention call on this thread
 * (kernel family, waves per workgroup, blocks per chunk, grid, partitions). */
const char* pkv_last_launch(void);

/*
 * kv_append -- write the step's new K/V token of every request into its pool
 * slot: for each request b and KV head g, the D elements k_new[b][g][:] and
 * v_new[b][g][:] are copied bit for bit to
 *   pool[block_tables[b][positions[b] / block_size]][g][positions[b] % block_size][:]
 * ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2, step
 * three: the block that a new token needs was allocated by the caller and is
 * already in the table).
 *
 *   dtype           storage dtype of k_new, v_new and the pools
 *   k_new, v_new    [B][H_kv][D], rows new_row_stride elements apart (>= H_kv*D)
 *   k_pool, v_pool  the pools, written in place
 *   block_tables    [B][bt_stride]
 *   positions       [B]; a request with positions[b] outside [0, bt_stride*block_size)
 *                   or whose target block id is outside [0, n_blocks) is skipped
 *   B               number of requests (0 is a no-op)
 * Two requests must not target the same (block, slot); if they do, which one
 * lands is unspecified.
 */
int pkv_kv_append(int dtype,
                  const void* k_new, const void* v_new, int64_t new_row_stride,
                  void* k_pool, void* v_pool,
                  const int32_t* block_tables, int32_t bt_stride,
                  const int32_t* positions,
                  int32_t B, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                  void* stream);

/*
 * Bytes of workspace pkv_paged_decode_attention needs for these sizes (0 when
 * the context is not split).  partition_size as below.
 */
size_t pkv_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t D,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * paged_decode_attention -- for every request b and query head h, with
 * g = h / (H_q / H_kv) and n = context_lens[b]:
 *   s_t = scale * <q[b][h][:], K_t>,  K_t, V_t the K/V rows of logical token t
 *         found through block_tables[b] as in kv_append, t = 0 .. n-1
 *   out[b][h][:] = sum_t softmax(s)_t * V_t            (float32; 0 when n == 0)
 *
 *   max_context_len  host-known upper bound on context_lens (sizes the grid;
 *                    no device-to-host copy is made).  Must be <= bt_stride*block_size.
 *   partition_size   0: each (request, KV head) is handled by one workgroup over
 *                    its whole context.  > 0: the context is cut into partitions
 *                    of this many tokens (a multiple of block_size), each
 *                    workgroup handles one partition and a log-sum-exp merge
 *                    kernel combines them in partition order (deterministic).
 *   workspace        device buffer of at least
 *                    pkv_decode_workspace_bytes(B, H_q, D, max_context_len,
 *                    partition_size) bytes, 256-byte aligned; may be NULL when
 *                    that is 0.  Its contents on entry do not matter.
 */
int pkv_paged_decode_attention(int dtype,
                               float* out,
                               const void* q, int64_t q_row_stride,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int32_t bt_stride,
                               const int32_t* context_lens,
                               int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                               int32_t block_size, int32_t n_blocks,
                               int32_t max_context_len, float scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * append_decode_attention -- one whole decode step: the new token of request
 * b is written at positions[b] exactly as kv_append does, and the query then
 * attends over the n_b = positions[b] + 1 tokens 0 .. positions[b], the new
 * one included ("Disaggregated LLM Serving：从 PD 分离到 Attention 卸载",
 * section 1: a decode step appends the new token's KV and reads the whole
 * history).  The workgroup that owns the new token reads it from k_new/v_new
 * and also writes it to the pool, so the step is one attention launch (plus
 * the merge when split) and the slot's previous contents are never read.
 *
 *   positions        [B]; n_b = positions[b] + 1 must lie in [1, max_context_len],
 *                    else that request gets a NaN output row and nothing is written
 *   other arguments  as in pkv_kv_append and pkv_paged_decode_attention
 *                    (the workspace size is the same as for paged_decode_attention)
 */
int pkv_append_decode_attention(int dtype,
                                float* out,
                                const void* q, int64_t q_row_stride,
                                const void* k_new, const void* v_new, int64_t new_row_stride,
                                void* k_pool, void* v_pool,
                                const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* positions,
                                int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                int32_t block_size, int32_t n_blocks,
                                int32_t max_context_len, float scale, int32_t partition_size,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * probe_stream_read -- measurement aid, not part of the decode step: reads
 * `bytes` bytes (rounded down to a multiple of 16) of device memory at `buf`
 * once with 16-byte loads from `grid` workgroups of 256 threads, so that the
 * HBM read bandwidth the device sustains can be timed next to the decode
 * kernels.  `sink` is a device word that is written only if the loaded data
 * fold to one particular value.  buf 16-byte aligned; 1 <= grid <= 2^20.
 */
int pkv_probe_stream_read(const void* buf, size_t bytes, void* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
