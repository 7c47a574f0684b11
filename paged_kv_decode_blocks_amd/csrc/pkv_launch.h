// pkv_launch.h -- host-side launchers of the gfx950 kernels (internal to libpkv).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"

namespace pkv {

struct AppendArgs {
    const char* k_new;
    const char* v_new;
    char* k_pool;
    char* v_pool;
    const int32_t* block_tables;
    const int32_t* positions;
    int64_t new_row_stride;   // elements
    int32_t bt_stride;
    int32_t B, H_kv, D, elem_bytes, n_blocks;
};

struct MergeArgs {
    float* out;
    const float* part_o;
    const float* part_lse;
    const int32_t* context_lens;   // plain call
    const int32_t* positions;      // fused call (n = positions + 1); context_lens unused
    int32_t BH, H_q, n_parts, part_tokens, max_context_len;
    const int32_t* even_meta;      // even split (see AttnArgs): pieces instead of partitions
    int32_t H_kv;                  // even split only
};

// pool[dst[i]] = pool[src[i]] for both pools; a block is block_bytes contiguous bytes
struct CopyArgs {
    char* k_pool;
    char* v_pool;
    const int32_t* src;
    const int32_t* dst;
    int64_t block_bytes;
    int32_t n, n_blocks;
};
constexpr int kCopyPieceBytes = 4096;   // bytes one 256-thread workgroup moves per piece

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);

// FP8 (OCP E4M3) K/V cache: one power-of-two scale per (block, KV head, slot).
struct AppendFp8Args {
    const char* k_new;          // source rows, src dtype
    const char* v_new;
    uint8_t* k_pool;
    uint8_t* v_pool;
    float* k_scale;
    float* v_scale;
    const int32_t* block_tables;
    const int32_t* positions;
    int64_t new_row_stride;     // elements
    int32_t bt_stride;
    int32_t B, H_kv, n_blocks;
};
hipError_t launch_kv_append_fp8(int src_dtype, int D, const AppendFp8Args& a, hipStream_t stream);
// MXFP4 pools: codes [n_blocks][H_kv][16][D/2] bytes, E8M0 scales [n_blocks][H_kv][16][D/32] bytes
struct AppendMx4Args {
    const char* k_new;          // source rows, src dtype
    const char* v_new;
    uint8_t* k_pool;
    uint8_t* v_pool;
    uint8_t* k_scale;
    uint8_t* v_scale;
    const int32_t* block_tables;
    const int32_t* positions;
    int64_t new_row_stride;     // elements
    int32_t bt_stride;
    int32_t B, H_kv, n_blocks;
};
hipError_t launch_kv_append_mxfp4(int src_dtype, int D, const AppendMx4Args& a, hipStream_t stream);
// per query head over MXFP4 pools (no append inside: lengths from context_lens, or
// positions + 1 when context_lens is NULL, after the append kernel has run)
hipError_t launch_decode_mxfp4(int q_dtype, int D, int nw, int ch, const AttnArgs& a, unsigned grid,
                               hipStream_t stream);
bool mxfp4_variant_exists(int nw, int ch);
// grouped MXFP4 attention on MFMA (f16/bf16 q, G <= 16): grid = n_parts * B * H_kv / hg;
// nw waves per workgroup, pf blocks in flight per wave, hg KV heads per workgroup (hg
// divides H_kv and nw)
hipError_t launch_decode_mxfp4_mfma(int q_dtype, int D, int nw, int pf, int hg, const AttnArgs& a, unsigned grid,
                                    hipStream_t stream);
bool mxfp4_mfma_variant_exists(int nw, int pf, int hg);
// grouped MXFP4 attention over an even split of the batch (a.even_waves, a.even_meta set):
// grid = ceil-runs * H_kv / nw workgroups of nw waves, one KV head per wave (nw divides H_kv)
hipError_t launch_decode_mxfp4_even(int q_dtype, int D, int nw, int pf, const AttnArgs& a, unsigned grid,
                                    hipStream_t stream);
bool mxfp4_even_variant_exists(int nw, int pf);
// resident workgroups per CU of that kernel (0 if the runtime cannot say)
int mxfp4_even_wgs_per_cu(int q_dtype, int D, int nw, int pf, int G, bool fused);
// per query head; q (and new rows) in q_dtype, K/V codes + scales in the AttnArgs pools
hipError_t launch_decode_fp8(int q_dtype, int D, int nw, int ch, int pf, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream);
bool fp8_variant_exists(int nw, int ch, int pf);
// grouped heads on MFMA over FP8 pools (no append inside; lengths from context_lens, or positions + 1 when
// context_lens is NULL)
// wpe: waves per SIMD the kernel's register allocation targets (2 or 3);
// kd: 1 = K tiles staged through LDS by DMA, 0 = K loaded straight into registers
hipError_t launch_decode_gqa_fp8(int q_dtype, int D, int nw, int ch, int pf, int wpe, int kd, const AttnArgs& a,
                                 unsigned grid, hipStream_t stream);
bool gqa_fp8_variant_exists(int nw, int ch, int pf, int wpe, int kd);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_decode_mha(int dtype, int D, int nw, int ch, int pf, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream);
// persistent per-head kernel: `grid` workgroups of 16 waves walk all units (one CU each)
hipError_t launch_decode_mha_persistent(int dtype, int D, bool append, const AttnArgs& a, unsigned grid,
                                        hipStream_t stream);
// kind 0: K/V through registers (nw, ch, pf = chunks in flight); kind 1: K/V through an LDS ring
// (nw, ch = 1, pf = ring slots per wave)
hipError_t launch_decode_gqa(int dtype, int D, int kind, int nw, int ch, int pf, bool append, const AttnArgs& a,
                             unsigned grid, hipStream_t stream);
hipError_t launch_lse_merge(int D, const MergeArgs& a, hipStream_t stream);
// even split of a grouped 16-bit batch: grid = ceil(a.even_waves / nw) workgroups of nw waves, pf blocks
// ahead per wave; then launch_lse_merge with m.even_meta set
hipError_t launch_decode_gqa_even(int dtype, int D, int nw, int pf, bool append, const AttnArgs& a, unsigned grid,
                                  hipStream_t stream);
bool gqa_even_variant_exists(int nw, int pf);
// workgroups of that variant resident on one CU of the current device (0 on error)
int gqa_even_wgs_per_cu(int dtype, int D, int nw, int pf, bool append);
hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t stream);
// reads of [n_blocks][heads][tile] K/V pools (and [..][64] scale pools) in a decode kernel's pattern
struct TileReadArgs {
    const char* k_pool;
    const char* v_pool;
    const char* k_scale;   // both scale pools, or neither (scales = 0)
    const char* v_scale;
    const int32_t* ids;    // [n_items] block ids; one outside [0, n_blocks) reads block 0
    unsigned* sink;
    int32_t n_blocks, heads, n_items, scales;
};
bool tile_read_variant_exists(int tile_bytes, int paths, int team, int depth);
// `grid` workgroups of 4 waves; teams of `team` waves; `paths` bit 1 K, 2 V, 4 scales by DMA into LDS;
// `depth` items in flight per wave
hipError_t launch_tile_read(const TileReadArgs& a, int tile_bytes, int paths, int team, int depth, int grid,
                            hipStream_t stream);
// `grid` 16-wave workgroups, one per CU, each running bf16 MFMA chains for `iterations` rounds
hipError_t launch_mfma_burn(int grid, int iterations, unsigned* sink, hipStream_t stream);
struct GemmArgs {
    const char* a;   // [M][K] bf16
    const char* b;   // [N][K] bf16 (B transposed)
    float* c;        // [M][N]
    int32_t M, N, K;
};
hipError_t launch_gemm_nt_bf16(int grid, const GemmArgs& g, hipStream_t stream);
bool mha_variant_exists(int nw, int ch, int pf);
bool gqa_variant_exists(int kind, int nw, int ch, int pf);

}  // namespace pkv
