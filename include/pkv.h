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
 * that point.  No compute entry point allocates device memory (only
 * pkv_decoder_create allocates, for its own metadata buffers), and calls on
 * different streams may overlap freely as long as their outputs do not alias.
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
    PKV_ERR_ALIASED_APPEND = -5,/* two appends of one step target the same (block, slot)
                                   (pkv_check_step_metadata, or any append entry point
                                   with PKV_DEBUG_CHECKS=1 in the environment)           */
    PKV_ERR_HIP = -6,           /* the HIP runtime reported an error when launching      */
    PKV_ERR_OUT_OF_BLOCKS = -7, /* block manager: too few free blocks                     */
    PKV_ERR_SEQUENCE = -8       /* block manager: sequence id unknown, or already in use  */
} pkv_status;

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Human-readable name of a pkv_status value. */
const char* pkv_status_string(int status);

/* Detail of the last non-OK return on this thread ("" if none). */
const char* pkv_last_error(void);

/* Launch geometry of the last successful attention call on this thread
 * (kernel family, waves per workgroup, blocks per chunk, grid, partitions).
 *
 * The launch shapes are the library's measured defaults.  For tuning only, they
 * can be overridden per process with environment variables read at each call:
 * PKV_MHA_{NW,CH,PF} (per-head 16-bit), PKV_GQA_{KIND,NW,CH,PF} (grouped 16-bit;
 * KIND 0 = K in registers, 1 = K and V through LDS, 2 = K through LDS),
 * PKV_FP8_{NW,CH,PF} (per-head FP8), PKV_GQA8_{NW,CH,PF,WPE,KDMA} (grouped
 * FP8) and PKV_MX4_{KIND,NW,CH,PF,HG} (MXFP4; KIND 0 = per query head on the
 * vector units, 1 = grouped heads on MFMA; CH for kind 0, PF and HG -- KV heads
 * per workgroup -- for kind 1).
 * Split steps: PKV_GQA_EVEN (grouped 16-bit with K in LDS) and PKV_MX4_EVEN
 * (grouped MXFP4): 0 = one workgroup per partition or span of partitions, 1 = the
 * even split of the batch's blocks into equal runs where the plan finds it pays,
 * 2 = wherever it applies; with PKV_GQA_EVEN_{NW,PF} and PKV_MX4_EVEN_{NW,PF};
 * PKV_PART_REV (0 = deal partitions first to last instead of last to first; the
 * results are bit-identical); PKV_LP_MIN_PART (the grouped FP8 and MXFP4 kernels'
 * smallest partition in tokens, 2048 by default, 0 = the caller's).  A combination
 * the library does not instantiate falls back to the default; results agree to the
 * same tolerance for every instantiated shape. */
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
 * Two requests must not target the same (block, slot): each new token has a
 * slot of its own (same section).  The kernels do not detect it (which write
 * lands is then unspecified); pkv_check_step_metadata does, and so does every
 * append entry point when PKV_DEBUG_CHECKS=1 is set in the environment.
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
 *                    of this many tokens (a multiple of block_size); each
 *                    partition's softmax state (maximum, sum, weighted V) is
 *                    computed on its own and the states are combined by a
 *                    log-sum-exp merge in partition order (deterministic).  The
 *                    16-bit kernels give a workgroup several consecutive
 *                    partitions, one per wave, and merge those themselves; a merge
 *                    kernel combines the workgroups' results when a context needs
 *                    more than one workgroup.
 *   workspace        device buffer of at least
 *                    pkv_decode_workspace_bytes(B, H_q, D, max_context_len,
 *                    partition_size) bytes, 256-byte aligned (a size that always
 *                    suffices); may be NULL when that is 0, or when the call's
 *                    workgroups each span every partition of their contexts and
 *                    merge them themselves (a call that needs partials and gets
 *                    no or too small a workspace returns PKV_ERR_WORKSPACE).  Its
 *                    contents on entry do not matter.
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
 * check_step_metadata -- debugging aid, not for the hot path: checks a step's
 * device-side metadata against the contract the kernels assume, and returns the
 * first violation ("从 PagedAttention 到 Prefill-Decode 分离的深度解析",
 * section 2.2: a request's logical block j lives in physical block
 * block_tables[b][j], and every new token is given a slot of its own).
 *
 *   context_lens / positions  exactly one is non-NULL: lengths of an attention
 *                    call, or append positions (kv_append, or the fused step
 *                    with n_b = positions[b] + 1)
 *   max_context_len  the bound the call passes (0 with positions: a plain
 *                    kv_append, whose lengths are not checked)
 * Returns PKV_ERR_INVALID_ARG if a length lies outside [0, max_context_len]
 * ([1, ...] for a fused step) or beyond bt_stride*block_size, or a block id the
 * step reads or writes lies outside [0, n_blocks); else PKV_ERR_ALIASED_APPEND
 * if two appends target the same (block, slot); else PKV_OK.  Runs on `stream`
 * and waits for it (synchronous); allocates nothing (the verdict word is a
 * device variable of the library).  Calls on one GPU that overlap race on that
 * word.  O(B^2) comparisons.
 */
int pkv_check_step_metadata(const int32_t* block_tables, int32_t bt_stride,
                            const int32_t* context_lens, const int32_t* positions,
                            int32_t B, int32_t block_size, int32_t n_blocks,
                            int32_t max_context_len, void* stream);

/*
 * append_decode_attention_noalloc -- pkv_append_decode_attention for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The split-KV partials go to
 * a fixed array the library holds in device memory (one copy per GPU, kept
 * until the process ends) instead of a caller's workspace; the call allocates
 * nothing and otherwise behaves exactly as pkv_append_decode_attention (same
 * kernels, same launch, same results bit for bit).
 *
 *   arguments        as in pkv_append_decode_attention, without the workspace
 *   limit            pkv_decode_workspace_bytes(B, H_q, D, max_context_len,
 *                    partition_size) must not exceed PKV_NOALLOC_SCRATCH_BYTES
 *                    (32 MiB; e.g. B 32 x 64 heads x 16 partitions of D 128 takes
 *                    17 MB), else PKV_ERR_WORKSPACE and nothing is launched
 *   device           the GPU current on the calling thread, which must be the
 *                    device of `stream`
 *   concurrency      every call on one GPU shares that GPU's array: two calls
 *                    whose work overlaps on the device (different streams, or
 *                    graphs replayed concurrently) race on it; order them on
 *                    one stream.  Nothing in the array needs clearing between
 *                    calls (the merge reads only the partitions the same call
 *                    wrote).
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pkv_append_decode_attention_noalloc(int dtype,
                                        float* out,
                                        const void* q, int64_t q_row_stride,
                                        const void* k_new, const void* v_new, int64_t new_row_stride,
                                        void* k_pool, void* v_pool,
                                        const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* positions,
                                        int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                        int32_t block_size, int32_t n_blocks,
                                        int32_t max_context_len, float scale, int32_t partition_size,
                                        void* stream);

/*
 * append_decode_attention_persistent -- the same fused step on a bounded share
 * of the GPU ("Injecting Adrenaline into LLM Serving" review, section 3.3.1:
 * decode attention is memory-bound, so a fraction of the compute units already
 * draws most of the HBM bandwidth and the rest can serve other work).  The step
 * runs as `n_workgroups` persistent workgroups of 16 waves that walk the
 * (request, head, partition) units round-robin; one such workgroup fills the
 * register file of its compute unit, so the step occupies n_workgroups CUs (all
 * of them when n_workgroups >= the CU count) and leaves the others to work on
 * other streams.  Results agree with pkv_append_decode_attention to the same
 * tolerance (the wave count per unit differs, so the summation order does).
 *
 *   n_workgroups     in [1, 65536]; more than the number of units is clamped
 *   dtype            PKV_F16 or PKV_BF16, and H_q == H_kv (else PKV_ERR_UNSUPPORTED)
 *   other arguments  as in pkv_append_decode_attention
 */
int pkv_append_decode_attention_persistent(int dtype,
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
                                           int32_t n_workgroups,
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

/*
 * probe_tile_read -- measurement aid, not part of the decode step: the reads a
 * paged decode kernel makes of its KV cache, without the arithmetic, so that the
 * rate of a kernel's own access pattern can be timed next to the plain stream.
 * A request's history sits in fixed-size blocks of a shared pool at places its
 * page table gives ("从 PagedAttention 到 Prefill-Decode 分离的深度解析",
 * section 2.2); here the block ids are the caller's, random in a measurement.
 *   k_pool, v_pool    device, [n_blocks][heads][tile_bytes], 16-byte aligned.
 *   k_scale, v_scale  device, [n_blocks][heads][64 bytes], or both NULL (no
 *                     scale reads); 4-byte aligned.
 *   block_ids         device int32 [n_items]; an id outside [0, n_blocks) reads
 *                     block 0.
 *   team              1, 2 or 4 waves of one workgroup (4 waves, 256 threads)
 *                     take an item together: block block_ids[t] and the team's
 *                     neighbouring heads team (t mod heads/team) + 0 .. team-1,
 *                     one head per wave.  heads % team == 0.
 *   paths             bit 1: K tiles, bit 2: V tiles, bit 4: scale tiles go
 *                     global -> LDS (global_load_lds); otherwise register
 *                     loads.
 *   depth             items whose loads each wave has in flight at once.
 *                     Built: depth 4 with tile_bytes 1024, 2048, 4096 and paths
 *                     0, 1, 5, with 1024 and 2048 and paths 7, and with 1024
 *                     and paths 4, 6; depths 2 and 8 with tile_bytes 1024 and
 *                     paths 0, 4, 6, 7 (PKV_ERR_UNSUPPORTED otherwise).
 *   grid              1 .. 65536 workgroups; teams walk the items grid-stride.
 *   sink              device word written only if the loaded data fold to one
 *                     particular value.
 * Bytes read: n_items * team * (2 tile_bytes + 128 if scales).  n_items = 0
 * launches nothing.  Errors: PKV_ERR_NULL, PKV_ERR_INVALID_ARG (alignment,
 * ranges, team), PKV_ERR_UNSUPPORTED, PKV_ERR_HIP (launch).
 */
int pkv_probe_tile_read(const void* k_pool, const void* v_pool, const void* k_scale, const void* v_scale,
                        int32_t n_blocks, int32_t heads, int32_t tile_bytes, const int32_t* block_ids,
                        int32_t n_items, int32_t team, int32_t paths, int32_t depth, void* sink, int32_t grid,
                        void* stream);

/*
 * probe_mfma_burn -- measurement aid, not part of the decode step: a compute-
 * bound neighbour for the step on a share of the CUs ("Injecting Adrenaline
 * into LLM Serving" review, section 3.3.1: decode attention beside compute-bound
 * work).  Launches `n_workgroups` workgroups of 16 waves, each holding 100 KiB
 * of LDS so that nothing else of this library fits on its CU; every wave runs
 * bf16 MFMA chains (v_mfma_f32_16x16x32_bf16, 8 chains) for `iterations` rounds,
 * i.e. n_workgroups * 16 * iterations * 8 * 16384 flops.  Touches no memory but
 * `sink` (a device word, written only if the result hits one value).
 *   n_workgroups in [1, 65536], iterations in [1, 2^30], sink 4-byte aligned.
 */
int pkv_probe_mfma_burn(int32_t n_workgroups, int32_t iterations, void* sink, void* stream);

/*
 * probe_gemm_bf16 -- measurement aid, not part of the decode step: a neighbour
 * that streams its operands from HBM, standing in for the prefill GEMMs that
 * share the GPU with decode attention ("Injecting Adrenaline into LLM Serving"
 * review, section 3.3.1).  c[M][N] = a[M][K] . b_t[N][K]^T in bf16 with float32
 * accumulation on the matrix cores; `n_workgroups` persistent workgroups of 8
 * waves walk the 256 x 256 output tiles round-robin, each workgroup holding
 * 128 KiB of LDS and most of its CU's registers, so that the grid occupies
 * n_workgroups CUs and nothing of the persistent decode step fits beside it.
 * 2 M N K flops.  M, N multiples of 256, K a multiple of 64, all 16-byte aligned;
 * n_workgroups in [1, 65536].
 */
int pkv_probe_gemm_bf16(int32_t n_workgroups, const void* a, const void* b_t, float* c,
                        int32_t M, int32_t N, int32_t K, void* stream);

/*
 * ---------------------------------------------------------------------------
 * FP8 K/V cache
 * ---------------------------------------------------------------------------
 * A low-precision KV cache stores K/V in a few bits with fine-grained scales
 * and dequantizes them before attention ("从 PagedAttention 到 Prefill-Decode
 * 分离的深度解析", section 6.2); decode attention reads the whole history every
 * step, so one-byte codes halve its HBM traffic against f16/bf16.  Format:
 * OCP E4M3 codes (bias 7, no infinities, S.1111.111 = NaN, largest 448) with one
 * power-of-two float scale per token row and KV head:
 *   k_pool, v_pool   : [n_blocks][H_kv][block_size][D] uint8 codes
 *   k_scale, v_scale : [n_blocks][H_kv][block_size] float32
 * Quantizing a row x: E = max(floor(log2 max|x|) - 8, -126) (0 for a zero row),
 * scale = 2^E, code = nearest E4M3 value to x / scale (ties to even, magnitudes
 * above 448 clamped, sign kept); its value is code * scale.  Each row is
 * quantized on its own when it is appended.  Non-finite new K/V values are
 * outside the contract.  q, k_new and v_new keep their own dtype (q_dtype /
 * src_dtype: PKV_F32, PKV_F16 or PKV_BF16); out is float32.  Pools 16-byte
 * aligned, scale arrays 4-byte aligned; other rules as the calls above.  With
 * grouped heads (H_q > H_kv) and f16/bf16 q the products run on the matrix
 * cores over codes widened to q's type; otherwise attention runs per query
 * head.  Either way the fused call quantizes the new rows inside the attention
 * launch (the workgroup holding the new position writes them to the pools), so
 * the step is one launch (plus the merge when split).
 */

/* Quantize each request's new K/V rows into slot positions[b] of its block. */
int pkv_kv_append_fp8(int src_dtype,
                      const void* k_new, const void* v_new, int64_t new_row_stride,
                      uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                      const int32_t* block_tables, int32_t bt_stride,
                      const int32_t* positions,
                      int32_t B, int32_t H_kv, int32_t D,
                      int32_t block_size, int32_t n_blocks,
                      void* stream);

/* pkv_paged_decode_attention over FP8 pools (same arguments and workspace rule). */
int pkv_paged_decode_attention_fp8(int q_dtype,
                                   float* out,
                                   const void* q, int64_t q_row_stride,
                                   const uint8_t* k_pool, const uint8_t* v_pool,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* context_lens,
                                   int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                   int32_t block_size, int32_t n_blocks,
                                   int32_t max_context_len, float scale, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* pkv_append_decode_attention over FP8 pools: the new rows (q_dtype) are
 * quantized in the attention launch, written with their scales, and attended
 * to as stored. */
int pkv_append_decode_attention_fp8(int q_dtype,
                                    float* out,
                                    const void* q, int64_t q_row_stride,
                                    const void* k_new, const void* v_new, int64_t new_row_stride,
                                    uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale,
                                    const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* positions,
                                    int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                    int32_t block_size, int32_t n_blocks,
                                    int32_t max_context_len, float scale, int32_t partition_size,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * ---------------------------------------------------------------------------
 * MXFP4 K/V cache
 * ---------------------------------------------------------------------------
 * The same page's 4-bit cache with fine-grained block scales, in the OCP
 * microscaling format MXFP4 (OCP MX specification v1.0: blocks of 32 elements
 * share one E8M0 scale): a quarter of the f16/bf16 bytes plus one scale byte per
 * 32 elements.
 *   k_pool, v_pool   : [n_blocks][H_kv][block_size][D/2] uint8, E2M1 codes two
 *                      per byte (element 2k in the low nibble of byte k;
 *                      magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, sign in bit 3)
 *   k_scale, v_scale : [n_blocks][H_kv][block_size][D/32] uint8, E8M0 scale of
 *                      each 32-element block of a row (value 2^(s - 127),
 *                      s = 255 is NaN)
 * Quantizing a block of 32 values x: E = floor(log2 max|x|) - 2 clamped to
 * [-127, 127] (-127 for an all-zero block), s = E + 127, code = nearest E2M1
 * value to x / 2^E (ties to the even code, magnitudes above 6 saturating, sign
 * kept); its value is code * 2^E (exact in float32).  Each row is quantized on
 * its own when it is appended.  Non-finite new K/V values are outside the
 * contract.  q, k_new and v_new keep their own dtype (PKV_F32, PKV_F16 or
 * PKV_BF16); out is float32.  Pools 16-byte aligned; D in {64, 128}; code
 * pools of 1 TiB or more return PKV_ERR_UNSUPPORTED; other rules as the calls
 * above.  With grouped heads (H_q / H_kv in 2..16) and an f16/bf16 q, one
 * workgroup serves a KV head's query heads on MFMA tiles, reading each block
 * once; otherwise attention runs per query head on the vector units.  The fused
 * call quantizes the new rows inside the grouped attention launch (the
 * workgroup holding the new position writes them to the pools), and in a launch
 * of its own before the per-head one.
 */

/* Quantize each request's new K/V rows into slot positions[b] of its block. */
int pkv_kv_append_mxfp4(int src_dtype,
                        const void* k_new, const void* v_new, int64_t new_row_stride,
                        uint8_t* k_pool, uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale,
                        const int32_t* block_tables, int32_t bt_stride,
                        const int32_t* positions,
                        int32_t B, int32_t H_kv, int32_t D,
                        int32_t block_size, int32_t n_blocks,
                        void* stream);

/* pkv_paged_decode_attention over MXFP4 pools (same arguments and workspace rule). */
int pkv_paged_decode_attention_mxfp4(int q_dtype,
                                     float* out,
                                     const void* q, int64_t q_row_stride,
                                     const uint8_t* k_pool, const uint8_t* v_pool,
                                     const uint8_t* k_scale, const uint8_t* v_scale,
                                     const int32_t* block_tables, int32_t bt_stride,
                                     const int32_t* context_lens,
                                     int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                     int32_t block_size, int32_t n_blocks,
                                     int32_t max_context_len, float scale, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

/* pkv_append_decode_attention over MXFP4 pools: the new rows (q_dtype) are
 * quantized and written with their scales, then attended to as stored. */
int pkv_append_decode_attention_mxfp4(int q_dtype,
                                      float* out,
                                      const void* q, int64_t q_row_stride,
                                      const void* k_new, const void* v_new, int64_t new_row_stride,
                                      uint8_t* k_pool, uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale,
                                      const int32_t* block_tables, int32_t bt_stride,
                                      const int32_t* positions,
                                      int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                      int32_t block_size, int32_t n_blocks,
                                      int32_t max_context_len, float scale, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * ---------------------------------------------------------------------------
 * Block manager (host side): the paging lifecycle of the KV pool
 * ---------------------------------------------------------------------------
 * Physical blocks are handed out only when a sequence's next token needs one,
 * and return to one global free pool as soon as no sequence maps them any more
 * ("从 PagedAttention 到 Prefill-Decode 分离的深度解析", section 2.2, the third
 * step: allocation on demand, reclaim at request end).  Several sequences may
 * map the same physical blocks, e.g. a shared system prompt whose KV is
 * computed once (same page, section 2.3); such blocks carry a reference count.
 * A full block is never written again.  A sequence about to append into a
 * partly filled block that another sequence also maps is first moved to a
 * fresh private copy of that block (copy-on-write): the call reports the
 * (source, destination) pair and the caller copies the block on the device
 * (pkv_copy_blocks) before the append.  The tables and positions these calls
 * return are exactly the block_tables / positions arguments of the decode
 * calls above, prepared on the host before the step (the "Injecting Adrenaline
 * into LLM Serving" review, section 3.2.1, on moving metadata preparation off
 * the critical path).
 *
 * Allocation order is deterministic: the free block with the smallest key is
 * handed out first, where key(i) = i for shuffle_seed == 0 and otherwise
 * (splitmix64(shuffle_seed + (i + 1) * 0x9E3779B97F4A7C15), i) compared
 * lexicographically (splitmix64 = the output mix of Steele, Lea and Flood's
 * SplitMix generator).  A seeded order scatters each sequence over the pool.
 *
 * All block-manager calls are host-only and synchronous; a manager is not
 * thread-safe (one per scheduler thread).  A call that fails returns a negative
 * pkv_status, sets pkv_last_error() and leaves the manager unchanged.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* New manager over physical blocks 0 .. n_blocks-1, block_size tokens each
 * (n_blocks >= 1, 1 <= block_size).  Returns NULL on invalid sizes. */
pkv_block_manager* pkv_bm_create(int32_t n_blocks, int32_t block_size, uint64_t shuffle_seed);
/* Frees the manager (NULL is allowed). */
void pkv_bm_destroy(pkv_block_manager* bm);

/* Register sequence seq_id with num_tokens >= 0 tokens (its prompt) and give it
 * ceil(num_tokens / block_size) fresh blocks.  PKV_ERR_SEQUENCE if seq_id is in
 * use, PKV_ERR_OUT_OF_BLOCKS if the pool is short. */
int pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens);

/* Register seq_id with num_tokens tokens whose first prefix_tokens tokens equal
 * those of the live sequence prefix_id (prefix_tokens <= num_tokens and <= its
 * length).  The first prefix_tokens / block_size blocks (whole blocks only) are
 * mapped from prefix_id and shared; the rest are fresh.  *shared_tokens receives
 * the number of tokens the new sequence gets for free (a multiple of
 * block_size); the caller writes the KV of tokens shared_tokens .. num_tokens-1. */
int pkv_bm_add_sequence_shared(pkv_block_manager* bm, int64_t seq_id, int32_t num_tokens, int64_t prefix_id,
                               int32_t prefix_tokens, int32_t* shared_tokens);

/* child_id starts as an exact copy of the live sequence parent_id: same length,
 * same physical blocks, partly filled last block included (shared until one of
 * them appends into it). */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);

/* Reserve the slot of the sequence's next token: *position = its length before
 * the call, then the length grows by one.  A token that starts a block gets a
 * fresh block; a token that lands in a shared, partly filled block triggers the
 * copy-on-write above, with *cow_src / *cow_dst set to the old and new block
 * ids (both -1 when nothing must be copied).  Any out pointer may be NULL. */
int pkv_bm_append_token(pkv_block_manager* bm, int64_t seq_id, int32_t* position, int32_t* cow_src,
                        int32_t* cow_dst);

/* One decode step's metadata: pkv_bm_append_token for seq_ids[0..B) in that
 * order (ids must be distinct), then the batch's block tables after the append.
 *   tables    [B][bt_stride] int32, rows padded with -1
 *   positions [B] int32, the slot index each sequence's new token goes to
 *             (context length of the step = positions[b] + 1)
 *   cow_src, cow_dst  [B] int32 each; the first *n_cow entries are the block
 *             pairs to copy before the step's append (may be NULL when the
 *             caller knows no block is shared; then a needed copy is an error)
 * Members are checked in batch order before anything changes: an unknown id
 * gives PKV_ERR_SEQUENCE, a repeated id or a table that would exceed bt_stride
 * PKV_ERR_INVALID_ARG; only then PKV_ERR_OUT_OF_BLOCKS if the pool cannot serve
 * the whole batch. */
int pkv_bm_append_batch(pkv_block_manager* bm, const int64_t* seq_ids, int32_t B, int32_t* tables,
                        int32_t bt_stride, int32_t* positions, int32_t* cow_src, int32_t* cow_dst,
                        int32_t* n_cow);

/* Drop the sequence; blocks whose reference count reaches zero return to the pool. */
int pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);

/* Number of free blocks, or -1 for a NULL manager. */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);
/* Number of live sequences, or -1 for a NULL manager. */
int32_t pkv_bm_num_sequences(const pkv_block_manager* bm);
/* Length of the sequence in tokens, or -1 if unknown. */
int32_t pkv_bm_sequence_length(const pkv_block_manager* bm, int64_t seq_id);
/* Number of sequences mapping the block (0 = free), or -1 if out of range. */
int32_t pkv_bm_block_refcount(const pkv_block_manager* bm, int32_t block);

/* The sequence's block table: min(count, capacity) ids into table (may be NULL
 * when capacity is 0), the full count into *n_blocks. */
int pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq_id, int32_t* table, int32_t capacity,
                       int32_t* n_blocks);

/* Block tables and lengths of a batch without changing anything:
 * tables [B][bt_stride] (rows padded with -1), context_lens [B].
 * PKV_ERR_INVALID_ARG if a sequence has more than bt_stride blocks. */
int pkv_bm_batch_tables(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t B, int32_t* tables,
                        int32_t bt_stride, int32_t* context_lens);

/*
 * copy_blocks -- device copy of whole physical blocks, every KV head, K and V:
 * pool[dst[i]] = pool[src[i]] for i < n, as the block manager's copy-on-write
 * asks (pools laid out as above).  src and dst are device int32 arrays of n
 * entries; a pair with an id outside [0, n_blocks) is skipped, and no block may
 * be both a source and a destination in one call.  n == 0 launches nothing.
 * Stream-ordered like the decode calls.
 */
int pkv_copy_blocks(int dtype, void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int32_t n,
                    int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks, void* stream);

/* copy_blocks for an FP8 cache: the blocks' codes and their row scales (pools
 * and scale arrays 16-byte aligned). */
int pkv_copy_blocks_fp8(uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale, const int32_t* src,
                        const int32_t* dst, int32_t n, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                        void* stream);

/* copy_blocks for an MXFP4 cache: the blocks' code bytes ([n_blocks][H_kv][16][D/2])
 * and their E8M0 scale bytes ([n_blocks][H_kv][16][D/32]); pools and scale arrays
 * 16-byte aligned.  Same pair rules as pkv_copy_blocks. */
int pkv_copy_blocks_mxfp4(uint8_t* k_pool, uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale, const int32_t* src,
                          const int32_t* dst, int32_t n, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                          void* stream);

/*
 * ---------------------------------------------------------------------------
 * Step graphs: the decode step captured once per (batch, context) bucket
 * ---------------------------------------------------------------------------
 * Launching a step's kernels one by one costs host time that a small decode
 * batch cannot hide (the "Injecting Adrenaline into LLM Serving" review,
 * section 3.2.2: per-layer CPU time far above GPU time without graphs, fixed by
 * capturing graphs over a two-dimensional grid of batch capacities and
 * replaying the smallest one that fits).  A pkv_step_graphs object captures,
 * for every pair (batch capacity Bc, context capacity Cc) of the given lists,
 * one HIP graph of the step over fixed buffers:
 *     pkv_append_decode_attention with B = Bc, max_context_len = Cc
 * and, when copy buffers are given, a second one that first runs
 *     pkv_copy_blocks over cow_src/cow_dst[0 .. Bc)
 * pkv_step_graphs_launch(B, max_len, n_copies) replays the graph with the
 * smallest Bc >= B and the smallest Cc >= max_len, with the copy node only if
 * n_copies > 0, on the caller's stream.  Before each launch the
 * caller writes the step's data into the buffers (device memory, e.g. by an
 * async copy on the same or an earlier-synchronised stream):
 *   positions[b] for b < B, and -1 for B <= b < Bc (such a padding row reads and
 *   writes nothing in the pools and gets a NaN output row);
 *   block_tables rows b < B; copy pairs, unused entries -1 (skipped).
 * Buffers are sized for the largest capacities; workspace for the largest
 * bucket (pkv_decode_workspace_bytes(max Bc, H_q, D, max Cc, partition_size)).
 * With k_scale / v_scale set the pools are an FP8 cache (uint8 codes, as in the
 * FP8 calls above; dtype is then q's) and the graphs run the FP8 step; with
 * k_mx_scale / v_mx_scale set they are an MXFP4 cache and the graphs run the
 * MXFP4 step (at most one of the two pairs).
 * The buffers must stay allocated, at the same addresses, for the object's
 * lifetime.  Capture happens in pkv_step_graphs_create on a stream of its own;
 * launch is asynchronous and allocation-free.  Not thread-safe per object.
 */
typedef struct pkv_step_desc {
    int dtype;
    int32_t H_q, H_kv, D, block_size, n_blocks;
    float scale;
    int32_t partition_size;
    float* out;                                  /* [max Bc][H_q][D] float32           */
    const void* q;                               /* [max Bc] rows of q_row_stride      */
    int64_t q_row_stride;
    const void* k_new;                           /* [max Bc] rows of new_row_stride    */
    const void* v_new;
    int64_t new_row_stride;
    void* k_pool;                                /* [n_blocks][H_kv][block_size][D]    */
    void* v_pool;
    const int32_t* block_tables;                 /* [max Bc][bt_stride]                */
    int32_t bt_stride;
    const int32_t* positions;                    /* [max Bc]                           */
    const int32_t* cow_src;                      /* [max Bc] or NULL (no copy node)    */
    const int32_t* cow_dst;                      /* [max Bc] or NULL                   */
    void* workspace;
    size_t workspace_bytes;
    float* k_scale;                              /* FP8 pools: row scales (else NULL)  */
    float* v_scale;
    uint8_t* k_mx_scale;                         /* MXFP4 pools: E8M0 scale bytes (else NULL) */
    uint8_t* v_mx_scale;
} pkv_step_desc;

typedef struct pkv_step_graphs pkv_step_graphs;

/* Capture n_batch x n_ctx graphs (capacities > 0, each list strictly
 * increasing, max Cc <= bt_stride * block_size).  Returns NULL on an invalid
 * description or a HIP error (detail in pkv_last_error()).  Runs on the current
 * HIP device, which must be the one owning the buffers. */
pkv_step_graphs* pkv_step_graphs_create(const pkv_step_desc* desc, const int32_t* batch_caps, int32_t n_batch,
                                        const int32_t* ctx_caps, int32_t n_ctx);

/* Replay the smallest fitting graph on `stream`.  PKV_ERR_INVALID_ARG if B or
 * max_context_len exceeds the largest capacity, if n_copies exceeds the chosen
 * batch capacity, or if n_copies > 0 without copy buffers (nothing launched). */
int pkv_step_graphs_launch(pkv_step_graphs* g, int32_t B, int32_t max_context_len, int32_t n_copies, void* stream);

/* Frees the graphs (NULL is allowed).  Work already launched is not waited for. */
void pkv_step_graphs_destroy(pkv_step_graphs* g);

/*
 * Dual step graphs: a local and an offloaded attention batch in one step.  The
 * Adrenaline review (section 3.2.1) runs the decode instance's own attention
 * and the attention it offloaded at the same time, and (section 3.2.2) captures
 * graphs bucketed over both batch sizes.  A pkv_dual_step_graphs object takes two
 * step descriptions (each with its own q/new rows/pools/tables/positions/out and,
 * when split, its own workspace; no copy buffers) and captures, for every pair
 * (local capacity Lc, offloaded capacity Oc) of the lists, one graph running
 *     the local step with B = Lc and the offloaded step with B = Oc,
 * both with max_context_len = ctx_cap: as two parallel branches (parallel != 0)
 * or one after the other (parallel == 0, to measure what the overlap buys).  A
 * capacity of 0 (allowed as the first entry of a list) leaves that branch out.
 * pkv_dual_step_graphs_launch(B_local, B_off) replays the smallest fitting pair
 * (nothing, if both are 0); padding rows as for pkv_step_graphs.  Buffers stay
 * allocated for the object's lifetime; launch is asynchronous and
 * allocation-free; not thread-safe per object.  Both branches read HBM at close
 * to its rate, so running them side by side cannot beat the sum of their bytes
 * at that rate: on MI355X the parallel form gained 3% for a long GQA batch beside
 * a long MHA one and lost up to 17% for two short batches (the second branch
 * starts later, on another hardware queue, and the join costs a few
 * microseconds); pick the form by measuring the pair.
 */
typedef struct pkv_dual_step_graphs pkv_dual_step_graphs;

/* Capture n_local x n_off graphs (capacity lists >= 0 and strictly increasing,
 * ctx_cap <= bt_stride * block_size of both).  NULL on an invalid description or
 * a HIP error (detail in pkv_last_error()). */
pkv_dual_step_graphs* pkv_dual_step_graphs_create(const pkv_step_desc* local, const pkv_step_desc* offloaded,
                                                  const int32_t* local_caps, int32_t n_local,
                                                  const int32_t* off_caps, int32_t n_off, int32_t ctx_cap,
                                                  int parallel);

/* Replay the smallest fitting graph on `stream`.  PKV_ERR_INVALID_ARG if a batch
 * exceeds its largest capacity (nothing launched). */
int pkv_dual_step_graphs_launch(pkv_dual_step_graphs* g, int32_t B_local, int32_t B_off, void* stream);

/* Frees the graphs (NULL is allowed).  Work already launched is not waited for. */
void pkv_dual_step_graphs_destroy(pkv_dual_step_graphs* g);

/*
 * ---------------------------------------------------------------------------
 * Decoder: the decode loop's per-step host work in one call
 * ---------------------------------------------------------------------------
 * Ties the pieces above into the loop a decode instance runs every step: the
 * block manager reserves each sequence's next slot, the resulting positions,
 * copy pairs and block tables are written into a pinned buffer, and the copy of
 * that buffer to the device plus the step (copy-on-write, fused append +
 * attention, merge) are enqueued, the step on the caller's stream -- as one
 * step-graph replay when capacity lists are given, else call by call.  A step
 * that reads much K/V (>= 512 MiB) copies its metadata on a stream of the
 * decoder's own, overlapping the previous step; a short one copies in order
 * on the caller's stream, where a cross-stream dependency would cost more
 * than the copy.  Two
 * metadata sets alternate, so the host prepares step k+1 while the GPU runs
 * step k (the "Injecting Adrenaline into LLM Serving" review, section 3.2.1, on
 * preparing metadata ahead of the step, and section 3.2.2 on graphs).
 *
 * The caller owns q, k_new, v_new, out, the pools and the workspace (device
 * memory, fixed addresses for the decoder's lifetime) and, before each step,
 * writes row b of q / k_new / v_new for seq_ids[b].  pkv_decoder_create
 * allocates the decoder's own metadata buffers (pinned host and device memory)
 * and captures its graphs; pkv_decoder_step allocates nothing.
 */
typedef struct pkv_decoder_desc {
    int dtype;
    int32_t H_q, H_kv, D, block_size, n_blocks;
    float scale;
    int32_t partition_size;
    int32_t max_batch;                           /* rows of q, k_new, v_new and out    */
    int32_t bt_stride;                           /* longest context = bt_stride * block_size */
    float* out;
    const void* q;
    int64_t q_row_stride;
    const void* k_new;
    const void* v_new;
    int64_t new_row_stride;
    void* k_pool;
    void* v_pool;
    void* workspace;                             /* for max_batch rows and the longest context */
    size_t workspace_bytes;
    uint64_t shuffle_seed;                       /* block manager allocation order    */
    /* Step graphs: strictly increasing capacities whose last entries are
     * max_batch and bt_stride * block_size; n_batch_caps = 0 launches eagerly. */
    const int32_t* batch_caps;
    int32_t n_batch_caps;
    const int32_t* ctx_caps;
    int32_t n_ctx_caps;
    float* k_scale;                              /* FP8 pools: row scales (else NULL); dtype is q's */
    float* v_scale;
    uint8_t* k_mx_scale;                         /* MXFP4 pools: E8M0 scale bytes (else NULL); dtype is q's */
    uint8_t* v_mx_scale;
} pkv_decoder_desc;

typedef struct pkv_decoder pkv_decoder;

/* Returns NULL on an invalid description or a HIP error (pkv_last_error()).
 * Uses the current HIP device. */
pkv_decoder* pkv_decoder_create(const pkv_decoder_desc* desc);

/* Waits for the decoder's launched work, then frees it (NULL is allowed). */
void pkv_decoder_destroy(pkv_decoder* dec);

/* The decoder's block manager (owned by the decoder): register, fork and free
 * sequences through the pkv_bm_* calls between steps. */
pkv_block_manager* pkv_decoder_block_manager(pkv_decoder* dec);

/* One decode step for seq_ids[0 .. B), 0 <= B <= max_batch, enqueued on
 * `stream`.  Errors from the block manager (unknown or repeated id, full pool,
 * context beyond bt_stride * block_size) return before anything changes; a
 * later PKV_ERR_HIP leaves the sequences already advanced.  *n_copies (may be
 * NULL) receives the number of copy-on-write block copies the step made. */
int pkv_decoder_step(pkv_decoder* dec, const int64_t* seq_ids, int32_t B, void* stream, int32_t* n_copies);

/*
 * ---------------------------------------------------------------------------
 * CU-limited streams: decode attention on a share of the GPU
 * ---------------------------------------------------------------------------
 * Attention offloaded next to other work on the same GPU runs on a bounded
 * share of the GPU's SMs, since decode attention is bandwidth-bound and needs
 * only a fraction of them to draw most of the memory bandwidth (the
 * "Injecting Adrenaline into LLM Serving" review, section 3.3).  On MI355X the
 * mechanism is a stream with a compute-unit mask: kernels launched on it run
 * only on the selected CUs.  Every entry point above takes such a stream.
 */

/* Number of compute units of the current HIP device (256 on MI355X), or a
 * negative pkv_status. */
int pkv_device_cu_count(void);

/* Host-only helper: set in mask[0 .. n_words) the bits of `count` CUs out of
 * n_cus (bit i of word w = CU 32*w + i, the runtime's CU numbering).
 * layout 0 = the first `count` CUs; layout 1 = `count` CUs spread evenly over
 * all n_cus (CU floor(j * n_cus / count) for j < count).  All other bits are
 * cleared.  Requires 1 <= count <= n_cus <= 32 * n_words. */
int pkv_cu_mask(int32_t n_cus, int32_t count, int layout, uint32_t* mask, int32_t n_words);

/* Create a stream (default priority, non-blocking) whose kernels run only on
 * the CUs set in mask[0 .. n_words); *stream receives the hipStream_t.  The
 * caller destroys it with pkv_stream_destroy. */
int pkv_stream_create_cu_masked(const uint32_t* mask, int32_t n_words, void** stream);
int pkv_stream_destroy(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
