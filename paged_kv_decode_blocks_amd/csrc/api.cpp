// api.cpp -- the C ABI of libpkv (declared in include/pkv.h).
//
// Host-side only: argument validation, launch geometry and dispatch to the
// gfx950 kernels.  Nothing here synchronises, copies device memory to the host
// or allocates; every kernel is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "pkv.h"
#include "pkv_host.h"
#include "pkv_launch.h"

namespace {
thread_local char g_err[512] = "";
thread_local char g_launch[256] = "";
}  // namespace

namespace pkv {

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_err[0] = 0; }

}  // namespace pkv

namespace {

using pkv::fail;

int elem_bytes(int dtype) {
    switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    default: return 0;
    }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_int(const char* name, int fallback) {
    const char* v = getenv(name);
    if (!v || !*v) return fallback;
    return atoi(v);
}

constexpr int32_t kMaxContext = 1 << 24;   // keeps every token index well inside int32

struct Plan {
    int32_t part_tokens;
    int32_t n_parts;
    bool grouped;     // matrix-core path (one workgroup per KV head and G query heads)
    int kind;         // grouped path: 0 = loads through registers, 1 = through an LDS ring
    int nw, ch, pf;   // waves per workgroup, blocks per chunk, chunks (or ring slots) in flight per wave
    int32_t wave_tokens;  // grouped kernel: > 0 = each wave streams one partition of this many tokens
    int32_t even_waves;   // grouped kernel: > 0 = even split of the batch over at most this many waves
    int wpe;          // grouped FP8 kernel: waves per SIMD its registers are sized for
    int kd;           // grouped FP8 kernel: K tiles staged through LDS (1) or loaded into registers (0)
    int hg;           // grouped MXFP4 kernel: KV heads per workgroup
    unsigned grid;
    size_t ws_o, ws_lse, ws_total;
};

int32_t coarsen_partitions(Plan& p, int32_t B, int32_t H_kv, int32_t max_ctx, int32_t partition_size,
                           int min_wgs_per_cu);

// Waves of the even-split kernel variant resident on the current device at once
// (occupancy per CU times CUs), cached per device; 0 if the runtime cannot say.
int64_t even_resident_waves(int dtype, int32_t D, int nw, int pf, bool fused) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int, int, bool>, int64_t> cache;
    const auto key = std::make_tuple(dev, dtype, (int)D, nw, pf, fused);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    const int64_t w = (int64_t)pkv::gqa_even_wgs_per_cu(dtype, D, nw, pf, fused) * cus * nw;
    cache[key] = w;
    return w;
}

// Launch geometry.  Unsplit: one partition spanning the padded context.
// `spans`: the kernel the plan is for implements one partition per wave (the 16-bit
// per-head and grouped kernels, not the persistent, FP8 or MXFP4 ones); `fused`: the
// call appends (picks the kernel instantiation whose occupancy sizes an even split).
Plan make_plan(int dtype, int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t max_ctx, int32_t partition_size,
               bool fp8 = false, bool spans = false, bool fused = false) {
    Plan p{};
    const int32_t padded = max_ctx <= 0 ? pkv::kBlockSize
                                        : (max_ctx + pkv::kBlockSize - 1) / pkv::kBlockSize * pkv::kBlockSize;
    if (partition_size <= 0 || partition_size >= padded) {
        p.part_tokens = padded;
        p.n_parts = 1;
    } else {
        p.part_tokens = partition_size;
        p.n_parts = (max_ctx + partition_size - 1) / partition_size;
    }
    const int32_t G = H_q / H_kv;
    p.grouped = G > 1 && dtype != PKV_F32;
    const int32_t blocks = p.part_tokens / pkv::kBlockSize;
    // Waves per workgroup and blocks per chunk, from launch-shape sweeps on MI355X:
    // when the grid already holds several workgroups per CU (split contexts, large
    // batches) small 4-wave workgroups let a CU overlap several workgroups' load
    // latency; a long unsplit context per workgroup spreads over more waves.
    const int64_t wgs = (int64_t)p.n_parts * B * (p.grouped ? H_kv : H_q);
    if (fp8 && p.grouped) {
        // 4-wave workgroups, one block ahead per wave, K staged through LDS (whose slots also
        // hold the closing merge: 35.6 KB, three workgroups per CU).  Against 2-wave ones on
        // MI355X (8 KV heads, 64 query heads, D = 128, bf16 q; variants interleaved): 32 x
        // 4096-16384 +2.3 %, 64 x 1024-8192 +3.8 %, 128 x 512-4096 +5.8 %, 4 x 4096-16384
        // +26 %, 32 x 2048-8192 +0.8 %; 16 x 4096-16384 -0.7 %, 64 x 2048 -1.0 %, 8 x
        // 4096-32768 -0.6 %.  Two or three blocks ahead were slower.
        p.kind = 2;   // grouped heads on MFMA over FP8 codes
        p.nw = env_int("PKV_GQA8_NW", 4);
        p.ch = env_int("PKV_GQA8_CH", 1);
        p.pf = env_int("PKV_GQA8_PF", 1);
        p.wpe = env_int("PKV_GQA8_WPE", 2);
        p.kd = env_int("PKV_GQA8_KDMA", 1);
        if (!pkv::gqa_fp8_variant_exists(p.nw, p.ch, p.pf, p.wpe, p.kd)) {
            p.nw = 4; p.ch = 1; p.pf = 1; p.wpe = 2; p.kd = 1;
        }
        p.grid = 0;   // after the partitions are final (below)
    } else if (fp8) {
        // launch-shape sweep on MI355X (c3-shaped FP8 batch): 4-wave workgroups with 2-block
        // chunks beat 8 waves (the decode work per byte keeps register use high) and deeper pipelines
        const int nw = 4, ch = 2, pf = 1;
        p.nw = env_int("PKV_FP8_NW", nw);
        p.ch = env_int("PKV_FP8_CH", ch);
        p.pf = env_int("PKV_FP8_PF", pf);
        if (!pkv::fp8_variant_exists(p.nw, p.ch, p.pf)) { p.nw = nw; p.ch = ch; p.pf = pf; }
        p.grid = (unsigned)wgs;
    } else if (p.grouped) {
        // measured on c5-shaped batches: K tiles staged through LDS by DMA (whole cache
        // lines) with V in registers beat K loaded into registers (half lines) by ~7 %;
        // 4-wave workgroups, one block per chunk, one chunk in flight
        p.kind = env_int("PKV_GQA_KIND", 2);
        p.nw = env_int("PKV_GQA_NW", 4);
        p.ch = env_int("PKV_GQA_CH", 1);
        p.pf = env_int("PKV_GQA_PF", 1);
        if (!pkv::gqa_variant_exists(p.kind, p.nw, p.ch, p.pf)) { p.kind = 2; p.nw = 4; p.ch = 1; p.pf = 1; }
        // A split step over a batch of mixed lengths: the even split (kernel 1e) cuts the
        // batch's blocks into equal runs, one wave per (run, KV head), one resident round of
        // waves for the whole batch, nw runs (a super-run) per workgroup.  Its pieces and the
        // merge's prefix fit the split's workspace: pieces <= (super-runs + B) * H_kv, G rows
        // each, after B + 3 ints.
        const int even_nw = env_int("PKV_GQA_EVEN_NW", 4), even_pf = env_int("PKV_GQA_EVEN_PF", 1);
        if (spans && p.n_parts > 1 && p.kind == 2 && env_int("PKV_GQA_EVEN", 1) && B <= pkv::kEvenMaxBatch &&
            pkv::gqa_even_variant_exists(even_nw, even_pf)) {
            const int64_t worst = (int64_t)B * ((max_ctx + pkv::kBlockSize - 1) / pkv::kBlockSize);   // per head
            const int64_t cap = (((int64_t)B * H_q * p.n_parts - B - 3) / H_q - B) * even_nw;
            const int64_t need = (worst + pkv::kEvenMaxWaveBlocks - 1) / pkv::kEvenMaxWaveBlocks;
            const int64_t resident = even_resident_waves(dtype, D, even_nw, even_pf, fused) / H_kv;
            const int64_t want = std::max(resident * std::max(1, env_int("PKV_GQA_EVEN_ROUNDS", 1)), need);
            const int64_t runs = std::min(want, cap);
            // The even split takes batches whose worst case holds at least 64 blocks per run
            // (shorter runs pay their per-piece start-up and the merge launch: on MI355X 8
            // requests of 1-16 K tokens, 32 blocks per run, ran 5 % slower, 8 of 4-32 K, 64 per
            // run, 13 % faster, one or two requests of 32-128 K, 16-32 per run, 3-15 % slower),
            // room for 3/4 of a round of runs in the workspace, and contexts that the
            // nw-partition spans would need the merge kernel for anyway (when one span covers
            // every context they need none: 64 requests of 2048 tokens ran 86 vs 101 us that way).
            const bool spans_merge = (int64_t)max_ctx > (int64_t)p.nw * partition_size;
            const bool fits = (worst >= 64 * runs && 4 * runs >= 3 * want && spans_merge) ||
                              env_int("PKV_GQA_EVEN", 1) == 2;
            if (resident > 0 && fits && runs >= need && runs >= 1 && worst < (int64_t)1 << 30 &&
                runs * H_kv < (int64_t)1 << 30) {
                p.nw = even_nw;
                p.ch = 1;
                p.pf = even_pf;
                p.even_waves = (int32_t)(runs * H_kv);
                p.grid = (unsigned)((runs + even_nw - 1) / even_nw * H_kv);
            }
        }
        // A split context: one workgroup spans nw consecutive partitions and wave w streams
        // partition w alone, so each wave's softmax state is its partition's and the
        // workgroup's closing merge of the waves is the log-sum-exp merge of those
        // partitions; the merge kernel then combines spans.  Long per-wave streams and
        // nw times fewer partial rows (measured on c5-shaped batches: as fast as 4x larger
        // partitions shared round-robin).  Kernel 1 only, a span within one window of
        // block ids, whole chunks per partition.
        const int32_t span = p.nw * partition_size;
        if (!p.even_waves && spans && p.n_parts > 1 && p.kind != 1 && env_int("PKV_GQA_BLOCKED", 1) &&
            span <= pkv::kGqaSpanTokens && (partition_size / pkv::kBlockSize) % p.ch == 0) {
            p.wave_tokens = partition_size;
            p.part_tokens = span;
            p.n_parts = (max_ctx + span - 1) / span;
        }
        if (!p.even_waves) p.grid = (unsigned)((int64_t)p.n_parts * B * H_kv);
    } else {
        // a PF-deep load pipeline pays where a workgroup walks a long unsplit context
        int nw = 4, ch = 2, pf = 1;
        if (p.n_parts == 1 && wgs > 4 * 256 && blocks >= 64) { nw = 8; pf = 2; }
        // a split context takes one partition per wave below (8 waves while a span of
        // 8 partitions fits one window of block ids: c4 at P = 512 then needs no merge
        // kernel, 397 vs 426 us per step with 4 waves sharing each partition)
        const bool want_spans = spans && p.n_parts > 1 && env_int("PKV_MHA_BLOCKED", 1);
        if (want_spans && 8 * partition_size <= pkv::kMhaWindowTokens) nw = 8;
        p.nw = env_int("PKV_MHA_NW", nw);
        p.ch = env_int("PKV_MHA_CH", ch);
        p.pf = env_int("PKV_MHA_PF", pf);
        if (!pkv::mha_variant_exists(p.nw, p.ch, p.pf)) { p.nw = nw; p.ch = ch; p.pf = pf; }
        // f32 rows of 128 take 16 loads per 2-block chunk: deeper pipelines would spill
        if (dtype == PKV_F32 && D == 128) { p.ch = 2; p.pf = 1; }
        // A split context may also take one partition per wave, as on the grouped path
        // (the workgroup's closing merge of its waves is the log-sum-exp merge of nw
        // consecutive partitions); per-head kernels only while a span fits one window
        // of block ids and holds whole chunks.
        const int32_t span = p.nw * partition_size;
        if (want_spans && span <= pkv::kMhaWindowTokens && (partition_size / pkv::kBlockSize) % p.ch == 0) {
            p.wave_tokens = partition_size;
            p.part_tokens = span;
            p.n_parts = (max_ctx + span - 1) / span;
        }
        p.grid = (unsigned)((int64_t)p.n_parts * B * H_q);
    }
    if (p.n_parts > 1) {
        p.ws_o = align_up((size_t)B * H_q * p.n_parts * D * sizeof(float), 256);
        p.ws_lse = align_up((size_t)B * H_q * p.n_parts * sizeof(float), 256);
    }
    p.ws_total = p.ws_o + p.ws_lse;
    if (fp8 && p.grouped) {
        coarsen_partitions(p, B, H_kv, max_ctx, partition_size, 8);
        p.grid = (unsigned)((int64_t)p.n_parts * B * H_kv);
    }
    return p;
}

// Compute units of the current device (cached per device; 0 if the runtime cannot say).
int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    static std::mutex mu;
    static int cached[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!cached[dev]) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cached[dev] = cus;
    }
    return cached[dev];
}

// The grouped FP8 and MXFP4 kernels split at no less than a floor of tokens, 2048 by default
// (a multiple of the caller's partition: fewer, longer workgroups and fewer partial rows,
// which the caller's workspace holds).  Measured on MI355X with the caller's 1024 (512):
// grouped MXFP4 +5 % on c5-shaped batches, +12-24 % on 1-128 requests; grouped FP8 +3-6 % on
// c5-shaped batches but -10 % where the coarser grid drops below two rounds of its resident
// 2-wave workgroups, so there the floor needs min_wgs_per_cu workgroups per CU.  Returns the
// partition in force (0 = the caller's).
int32_t coarsen_partitions(Plan& p, int32_t B, int32_t H_kv, int32_t max_ctx, int32_t partition_size,
                           int min_wgs_per_cu) {
    const int32_t floor_tokens = env_int("PKV_LP_MIN_PART", 2048);
    if (p.n_parts <= 1 || floor_tokens <= partition_size) return 0;
    const int32_t k = (floor_tokens + partition_size - 1) / partition_size;
    const int64_t pt = (int64_t)k * partition_size;
    const int32_t n_parts = pt >= max_ctx ? 1 : (int32_t)((max_ctx + pt - 1) / pt);
    if (min_wgs_per_cu > 0 && (int64_t)n_parts * B * H_kv < (int64_t)min_wgs_per_cu * device_cus()) return 0;
    if (n_parts == 1) {
        p.part_tokens = (max_ctx + pkv::kBlockSize - 1) / pkv::kBlockSize * pkv::kBlockSize;
    } else {
        p.part_tokens = (int32_t)pt;
    }
    p.n_parts = n_parts;
    return (int32_t)pt;
}

// Workgroups of the grouped MXFP4 even-split kernel resident on the current device at
// once (occupancy per CU times CUs), cached per device; 0 if the runtime cannot say.
int64_t mx4_even_resident_wgs(int dtype, int32_t D, int nw, int pf, int G, bool fused) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int, bool, bool>, int64_t> cache;
    const auto key = std::make_tuple(dev, dtype * 1000 + (int)D, nw, pf, G <= 8, fused);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    const int64_t n = (int64_t)pkv::mxfp4_even_wgs_per_cu(dtype, D, nw, pf, G, fused) * cus;
    cache[key] = n;
    return n;
}

// The grouped MXFP4 kernel's even split of a split step: the batch's blocks cut into
// equal runs, a workgroup per (run, group of nw KV heads), one resident round (the runs
// are sized so that a run is at most kEvenMaxWaveBlocks blocks and the pieces, ids
// (run + request) H_kv + head, fit the caller's workspace).  PKV_MX4_EVEN: 0 never,
// 2 whenever it fits, 1 (default) when the gate below holds; PKV_MX4_EVEN_NW / _PF pick
// the variant (default 4 KV heads per workgroup, else 2 with two chunks in flight).
// Returns whether the plan took it (p: nw, pf, hg, even_waves, grid).
//
// Gate, from MI355X against the per-partition kernel at its 2048-token floor (8 KV heads,
// 64 query heads, D = 128, bf16 q, 4-head workgroups; ctx uniform in the range; variants
// interleaved): 48 x 4096-16384 +6.2 %, 64 x 1024-8192 +2.2 %, 24 x 8192-32768 +0.5 %,
// 32 x 4096-16384 -0.2 %; 128 x 512-4096 -2.2 %, 32 x 2048-8192 -8 %, 16 x 4096-16384
// -17 % (8-head workgroups 0-3 % behind 4-head ones).  The losing batches' worst case (B
// requests of the longest context) is 64 blocks per run of one resident round, or their
// contexts are short; the others' 125 or more.  So: 4-head workgroups, a worst case of at
// least 96 blocks per run, and a longest context of at least 8192 tokens.
bool mx4_even_plan(Plan& p, int dtype, int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t max_ctx,
                   bool fused) {
    const int mode = env_int("PKV_MX4_EVEN", 1);
    if (!mode || p.n_parts <= 1 || B < 1 || B > pkv::kEvenMaxBatch) return false;
    const int nw = env_int("PKV_MX4_EVEN_NW", H_kv % 4 == 0 ? 4 : 2);
    const int pf = env_int("PKV_MX4_EVEN_PF", nw == 2 ? 2 : 1);
    if (nw <= 0 || H_kv % nw || !pkv::mxfp4_even_variant_exists(nw, pf)) return false;
    const int64_t worst = (int64_t)B * ((max_ctx + pkv::kBlockSize - 1) / pkv::kBlockSize);   // blocks per KV head
    const int64_t cap = ((int64_t)B * H_q * p.n_parts - B - 3) / H_q - B;                    // runs whose pieces fit
    const int64_t need = (worst + pkv::kEvenMaxWaveBlocks - 1) / pkv::kEvenMaxWaveBlocks;
    const int64_t resident = mx4_even_resident_wgs(dtype, D, nw, pf, H_q / H_kv, fused) / (H_kv / nw);
    const int64_t runs = std::min(std::max(resident, need), cap);
    const bool fits = mode == 2 || (nw == 4 && pf == 1 && worst >= 96 * runs && max_ctx >= 8192);
    if (resident <= 0 || runs < need || runs < 1 || worst >= (int64_t)1 << 30 || !fits) return false;
    p.nw = nw;
    p.pf = pf;
    p.hg = nw;
    p.even_waves = (int32_t)(runs * H_kv);
    p.grid = (unsigned)(runs * (H_kv / nw));
    return true;
}

int check_common(int dtype, int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                 int32_t bt_stride, int32_t max_ctx, int32_t partition_size) {
    if (!elem_bytes(dtype)) return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not one of PKV_F32/F16/BF16", dtype);
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B = %d is negative", B);
    if (H_q <= 0 || H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_q = %d, H_kv = %d must be positive", H_q, H_kv);
    if (H_q % H_kv) return fail(PKV_ERR_INVALID_ARG, "H_q = %d is not a multiple of H_kv = %d", H_q, H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride = %d must be positive", bt_stride);
    if (max_ctx < 0 || max_ctx > kMaxContext)
        return fail(PKV_ERR_INVALID_ARG, "max_context_len = %d outside [0, %d]", max_ctx, kMaxContext);
    if ((int64_t)max_ctx > (int64_t)bt_stride * block_size)
        return fail(PKV_ERR_INVALID_ARG, "max_context_len = %d exceeds bt_stride*block_size = %lld", max_ctx,
                    (long long)bt_stride * block_size);
    if (partition_size < 0 || partition_size % block_size)
        return fail(PKV_ERR_INVALID_ARG, "partition_size = %d must be 0 or a positive multiple of %d",
                    partition_size, block_size);
    const int32_t G = H_q / H_kv;
    if (G > 16 && dtype != PKV_F32)
        return fail(PKV_ERR_UNSUPPORTED, "G = H_q/H_kv = %d (the grouped path takes up to 16)", G);
    return PKV_OK;
}

int check_stride(const char* name, int64_t stride, int64_t min_elems, int eb) {
    if (stride < min_elems)
        return fail(PKV_ERR_INVALID_ARG, "%s = %lld is smaller than %lld", name, (long long)stride, (long long)min_elems);
    if ((stride * eb) % 16)
        return fail(PKV_ERR_INVALID_ARG, "%s = %lld elements is not a multiple of 16 bytes", name, (long long)stride);
    return PKV_OK;
}

struct Fp8Scales {
    const float* k;
    const float* v;
    float* k_w;
    float* v_w;
};

struct Mx4Scales {   // E8M0 scale bytes of MXFP4 pools
    const uint8_t* k;
    const uint8_t* v;
    uint8_t* k_w;
    uint8_t* v_w;
};

int launch_attention(int dtype, float* out, const void* q, int64_t q_row_stride, const void* k_new, const void* v_new,
                     int64_t new_row_stride, const void* k_pool, const void* v_pool, void* k_pool_w, void* v_pool_w,
                     const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                     const int32_t* positions, int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t block_size,
                     int32_t n_blocks, int32_t max_ctx, float scale, int32_t partition_size, void* workspace,
                     size_t workspace_bytes, void* stream, const Fp8Scales* fp8 = nullptr,
                     int32_t persistent_wgs = 0, const Mx4Scales* mx4 = nullptr) {
    const bool fused = positions != nullptr;
    int st = check_common(dtype, B, H_q, H_kv, D, block_size, n_blocks, bt_stride, max_ctx, partition_size);
    if (st) return st;
    if (B == 0) return PKV_OK;
    const int eb = elem_bytes(dtype);
    if (!out || !q || !k_pool || !v_pool || !block_tables) return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (fused ? (!k_new || !v_new) : !context_lens) return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (fused && (!aligned16(k_new) || !aligned16(v_new))))
        return fail(PKV_ERR_INVALID_ARG, "q, out, k_new, v_new and the pools must be 16-byte aligned");
    if ((st = check_stride("q_row_stride", q_row_stride, (int64_t)H_q * D, eb))) return st;
    if (fused && (st = check_stride("new_row_stride", new_row_stride, (int64_t)H_kv * D, eb))) return st;
    if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
    if (fp8) {
        if (!fp8->k || !fp8->v) return fail(PKV_ERR_NULL, "k_scale and v_scale must not be NULL");
        if ((reinterpret_cast<uintptr_t>(fp8->k) | reinterpret_cast<uintptr_t>(fp8->v)) & 3u)
            return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
    }
    if (mx4 && (!mx4->k || !mx4->v)) return fail(PKV_ERR_NULL, "k_scale and v_scale must not be NULL");
    // the grouped MXFP4 kernel addresses blocks in 256-byte units held in 32 bits
    if (mx4 && (uint64_t)n_blocks * H_kv * block_size * (D / 2) >= (1ull << 40))
        return fail(PKV_ERR_UNSUPPORTED, "MXFP4 code pools of 1 TiB or more are not supported");

    // one partition per wave: the 16-bit per-head and grouped kernels implement it (on the
    // grouped FP8 kernel it measured slower: c5f8 0.602 vs 0.621 of 8 TB/s)
    Plan p = make_plan(dtype, B, H_q, H_kv, D, max_ctx, partition_size, fp8 != nullptr,
                       !fp8 && !mx4 && !persistent_wgs, fused);
    if (mx4) {
        // kind 1: one workgroup per KV head and its G <= 16 query heads on MFMA (f16/bf16 q),
        // reading each K/V block once for the group; kind 0: one workgroup per query head on the
        // vector units (any q dtype).  With one query head per KV head the MFMA tiles are 1/16
        // used and kind 0 is faster, so it is the default there.
        const bool mfma_ok = (dtype == PKV_F16 || dtype == PKV_BF16) && H_q / H_kv <= 16;
        p.kind = mfma_ok ? env_int("PKV_MX4_KIND", H_q > H_kv ? 1 : 0) : 0;
        if (p.kind != 0 && p.kind != 1) p.kind = 1;
        p.grouped = p.kind == 1;
        p.pf = 1;
        if (p.kind == 1) {   // blocks stream through an LDS ring, pf blocks ahead per wave
            p.nw = env_int("PKV_MX4_NW", 4);
            p.ch = 1;
            p.pf = env_int("PKV_MX4_PF", 1);
            p.hg = env_int("PKV_MX4_HG", 1);
            if (p.hg <= 0 || H_kv % p.hg) p.hg = 1;
            if (!pkv::mxfp4_mfma_variant_exists(p.nw, p.pf, p.hg)) { p.nw = 4; p.pf = 1; p.hg = 1; }
            if (!mx4_even_plan(p, dtype, B, H_q, H_kv, D, max_ctx, fused)) {
                coarsen_partitions(p, B, H_kv, max_ctx, partition_size, 0);
                p.grid = (unsigned)((int64_t)p.n_parts * B * (H_kv / p.hg));
            }
        } else {
            p.nw = env_int("PKV_MX4_NW", 4);
            p.ch = env_int("PKV_MX4_CH", 2);
            if (!pkv::mxfp4_variant_exists(p.nw, p.ch)) { p.nw = 4; p.ch = 2; }
            p.grid = (unsigned)((int64_t)p.n_parts * B * H_q);
        }
    }
    if ((int64_t)p.n_parts * B * (p.grouped ? H_kv : H_q) > 0x7fffffff)
        return fail(PKV_ERR_INVALID_ARG, "grid too large");
    if (persistent_wgs && (fp8 || p.grouped || (dtype != PKV_F16 && dtype != PKV_BF16)))
        return fail(PKV_ERR_UNSUPPORTED, "the persistent step takes f16/bf16 K/V with one query head per KV head");
    if (p.ws_total) {
        if (!workspace) return fail(PKV_ERR_WORKSPACE, "split needs %zu bytes of workspace, got NULL", p.ws_total);
        if (workspace_bytes < p.ws_total)
            return fail(PKV_ERR_WORKSPACE, "split needs %zu bytes of workspace, got %zu", p.ws_total, workspace_bytes);
        if (reinterpret_cast<uintptr_t>(workspace) & 255u)
            return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    }

    pkv::AttnArgs a{};
    a.out = out;
    a.part_o = p.ws_total ? reinterpret_cast<float*>(workspace) : nullptr;
    a.part_lse = p.ws_total ? reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + p.ws_o) : nullptr;
    a.q = reinterpret_cast<const char*>(q);
    a.k_pool = reinterpret_cast<const char*>(k_pool);
    a.v_pool = reinterpret_cast<const char*>(v_pool);
    a.k_pool_w = reinterpret_cast<char*>(k_pool_w);
    a.v_pool_w = reinterpret_cast<char*>(v_pool_w);
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.positions = positions;
    a.k_new = reinterpret_cast<const char*>(k_new);
    a.v_new = reinterpret_cast<const char*>(v_new);
    a.q_row_stride = q_row_stride;
    a.new_row_stride = new_row_stride;
    a.bt_stride = bt_stride;
    a.B = B;
    a.H_q = H_q;
    a.H_kv = H_kv;
    a.G = H_q / H_kv;
    a.n_blocks = n_blocks;
    a.max_context_len = max_ctx;
    a.part_tokens = p.part_tokens;
    a.n_parts = p.n_parts;
    a.wave_tokens = p.wave_tokens;
    // the last partitions first: measured on MI355X, c4 split every 256 tokens 400 vs 410 us,
    // c5 over four-partition spans 221 vs 226 us, c5f4 +1-3 %, the grouped FP8 kernel unchanged
    a.part_rev = env_int("PKV_PART_REV", 1) != 0;
    if (p.even_waves) {   // the lse area starts with the merge's prefix: [tw, waves, blocks before b (B + 1)]
        a.even_waves = p.even_waves;
        a.even_min_run = std::min(std::max(env_int("PKV_GQA_EVEN_MINRUN", pkv::kEvenMinWaveBlocks),
                                           pkv::kEvenMinWaveBlocks), pkv::kEvenMaxWaveBlocks);
        a.even_meta = reinterpret_cast<int32_t*>(a.part_lse);
        a.part_lse += B + 3;
    }
    a.scale_log2 = scale * pkv::kLog2e;
    if (fp8) {
        a.k_scale = fp8->k;
        a.v_scale = fp8->v;
        a.k_scale_w = fp8->k_w;
        a.v_scale_w = fp8->v_w;
    }
    if (mx4) {
        a.k_mx_scale = mx4->k;
        a.v_mx_scale = mx4->v;
        a.k_mx_scale_w = mx4->k_w;
        a.v_mx_scale_w = mx4->v_w;
    }

    if (fused) {
        st = pkv::debug_check_appends(block_tables, bt_stride, positions, B, block_size, n_blocks, max_ctx, stream);
        if (st) return st;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (mx4) {
        // the per-head kernel reads the new row from the pool: quantize it there first (the
        // grouped kernel quantizes it itself)
        if (fused && p.kind == 0) {
            pkv::AppendMx4Args ap{};
            ap.k_new = a.k_new;
            ap.v_new = a.v_new;
            ap.k_pool = reinterpret_cast<uint8_t*>(k_pool_w);
            ap.v_pool = reinterpret_cast<uint8_t*>(v_pool_w);
            ap.k_scale = mx4->k_w;
            ap.v_scale = mx4->v_w;
            ap.block_tables = block_tables;
            ap.positions = positions;
            ap.new_row_stride = new_row_stride;
            ap.bt_stride = bt_stride;
            ap.B = B;
            ap.H_kv = H_kv;
            ap.n_blocks = n_blocks;
            e = pkv::launch_kv_append_mxfp4(dtype, D, ap, s);
            if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append_mxfp4 launch: %s", hipGetErrorString(e));
        }
        e = p.kind == 1 && p.even_waves ? pkv::launch_decode_mxfp4_even(dtype, D, p.nw, p.pf, a, p.grid, s)
            : p.kind == 1                ? pkv::launch_decode_mxfp4_mfma(dtype, D, p.nw, p.pf, p.hg, a, p.grid, s)
                        : pkv::launch_decode_mxfp4(dtype, D, p.nw, p.ch, a, p.grid, s);
    } else if (fp8 && p.grouped) {
        // in the fused step the kernel quantizes and writes the new rows itself
        e = pkv::launch_decode_gqa_fp8(dtype, D, p.nw, p.ch, p.pf, p.wpe, p.kd, a, p.grid, s);
    } else if (fp8) {
        e = pkv::launch_decode_fp8(dtype, D, p.nw, p.ch, p.pf, fused, a, p.grid, s);
    } else if (p.grouped && p.even_waves) {
        e = pkv::launch_decode_gqa_even(dtype, D, p.nw, p.pf, fused, a, p.grid, s);
    } else if (p.grouped) {
        e = pkv::launch_decode_gqa(dtype, D, p.kind, p.nw, p.ch, p.pf, fused, a, p.grid, s);
    } else if (persistent_wgs) {
        e = pkv::launch_decode_mha_persistent(dtype, D, fused, a, std::min<unsigned>(p.grid, (unsigned)persistent_wgs),
                                              s);
    } else {
        e = pkv::launch_decode_mha(dtype, D, p.nw, p.ch, p.pf, fused, a, p.grid, s);
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
    if (p.n_parts > 1) {
        pkv::MergeArgs m{};
        m.out = out;
        m.part_o = a.part_o;
        m.part_lse = a.part_lse;
        m.context_lens = fused ? nullptr : context_lens;
        m.positions = positions;
        m.BH = B * H_q;
        m.H_q = H_q;
        m.n_parts = p.n_parts;
        m.part_tokens = p.part_tokens;
        m.max_context_len = max_ctx;
        m.even_meta = a.even_meta;
        m.H_kv = H_kv;
        e = pkv::launch_lse_merge(D, m, s);
        if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
    }
    if (mx4) {
        char hg[48] = "";
        if (p.kind == 1 && p.even_waves) snprintf(hg, sizeof hg, " hg=%d even_waves=%d", p.hg, p.even_waves);
        else if (p.kind == 1) snprintf(hg, sizeof hg, " hg=%d", p.hg);
        snprintf(g_launch, sizeof g_launch, "%s dtype=%d D=%d nw=%d ch=%d pf=%d%s grid=%u part_tokens=%d n_parts=%d%s",
                 p.kind == 1 ? (p.even_waves ? "mxfp4_mfma_even" : "mxfp4_mfma") : "mxfp4", dtype, D, p.nw, p.ch, p.pf,
                 hg, p.grid, p.part_tokens, p.n_parts, fused ? " fused_append" : "");
    } else if (persistent_wgs) {
        snprintf(g_launch, sizeof g_launch,
                 "mha_persistent dtype=%d D=%d nw=16 ch=%d pf=1 grid=%u units=%u part_tokens=%d n_parts=%d%s", dtype, D,
                 (dtype == PKV_BF16 && D == 128) ? 1 : 2, std::min<unsigned>(p.grid, (unsigned)persistent_wgs), p.grid,
                 p.part_tokens, p.n_parts, fused ? " fused_append" : "");
    } else {
        char wt[32] = "";
        if (p.wave_tokens) snprintf(wt, sizeof wt, " wave_tokens=%d", p.wave_tokens);
        if (p.even_waves) snprintf(wt, sizeof wt, " even_waves=%d", p.even_waves);
        snprintf(g_launch, sizeof g_launch, "%s dtype=%d D=%d nw=%d ch=%d pf=%d%s grid=%u part_tokens=%d n_parts=%d%s%s",
                 fp8 ? (p.grouped ? "gqa_mfma_fp8" : "fp8")
                     : p.grouped ? (p.even_waves ? "gqa_mfma_even"
                                   : p.kind == 1 ? "gqa_mfma_lds" : p.kind == 2 ? "gqa_mfma_kdma" : "gqa_mfma")
                                 : "mha",
                 dtype, D, p.nw, p.ch, p.pf,
                 (fp8 && p.grouped)
                     ? (p.kd ? (p.wpe == 3 ? " wpe=3 kdma" : " wpe=2 kdma") : (p.wpe == 3 ? " wpe=3" : " wpe=2"))
                     : "",
                 p.grid, p.part_tokens, p.n_parts, wt, fused ? " fused_append" : "");
    }
    g_err[0] = 0;
    return PKV_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch for the allocation-free fused step: the split-KV partials of
// pkv_append_decode_attention_noalloc live in this fixed device array.  Each GPU
// the library runs on holds its own copy, at its own address, until the process
// ends.  In host code the array's name is only a host-side stand-in: the device
// address comes from hipGetSymbolAddress, once per device, and only that address
// is ever handed to a kernel.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`, looked up on the first
// call on that device with the device current.
int scratch_for_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PKV_OK;
}
}  // namespace

extern "C" {

int pkv_version(void) { return 100; }

const char* pkv_status_string(int status) {
    switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_NULL: return "PKV_ERR_NULL";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_ALIASED_APPEND: return "PKV_ERR_ALIASED_APPEND";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    case PKV_ERR_SEQUENCE: return "PKV_ERR_SEQUENCE";
    default: return "PKV_UNKNOWN_STATUS";
    }
}

const char* pkv_last_error(void) { return g_err; }

const char* pkv_last_launch(void) { return g_launch; }

int pkv_kv_append(int dtype, const void* k_new, const void* v_new, int64_t new_row_stride, void* k_pool, void* v_pool,
                  const int32_t* block_tables, int32_t bt_stride, const int32_t* positions, int32_t B, int32_t H_kv,
                  int32_t D, int32_t block_size, int32_t n_blocks, void* stream) {
    const int eb = elem_bytes(dtype);
    if (!eb) return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not one of PKV_F32/F16/BF16", dtype);
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B = %d is negative", B);
    if (H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_kv = %d must be positive", H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride = %d must be positive", bt_stride);
    if (B == 0) return PKV_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !positions)
        return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKV_ERR_INVALID_ARG, "k_new, v_new and the pools must be 16-byte aligned");
    int st = check_stride("new_row_stride", new_row_stride, (int64_t)H_kv * D, eb);
    if (st) return st;
    pkv::AppendArgs a{};
    a.k_new = reinterpret_cast<const char*>(k_new);
    a.v_new = reinterpret_cast<const char*>(v_new);
    a.k_pool = reinterpret_cast<char*>(k_pool);
    a.v_pool = reinterpret_cast<char*>(v_pool);
    a.block_tables = block_tables;
    a.positions = positions;
    a.new_row_stride = new_row_stride;
    a.bt_stride = bt_stride;
    a.B = B;
    a.H_kv = H_kv;
    a.D = D;
    a.elem_bytes = eb;
    a.n_blocks = n_blocks;
    if ((st = pkv::debug_check_appends(block_tables, bt_stride, positions, B, block_size, n_blocks, 0, stream)))
        return st;
    hipError_t e = pkv::launch_kv_append(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append launch: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return PKV_OK;
}

int pkv_kv_append_fp8(int src_dtype, const void* k_new, const void* v_new, int64_t new_row_stride, uint8_t* k_pool,
                      uint8_t* v_pool, float* k_scale, float* v_scale, const int32_t* block_tables, int32_t bt_stride,
                      const int32_t* positions, int32_t B, int32_t H_kv, int32_t D, int32_t block_size,
                      int32_t n_blocks, void* stream) {
    const int eb = elem_bytes(src_dtype);
    if (!eb) return fail(PKV_ERR_UNSUPPORTED, "src_dtype %d is not one of PKV_F32/F16/BF16", src_dtype);
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B = %d is negative", B);
    if (H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_kv = %d must be positive", H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride = %d must be positive", bt_stride);
    if (B == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !positions)
        return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
        ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3u))
        return fail(PKV_ERR_INVALID_ARG, "rows and pools must be 16-byte aligned, scales 4-byte aligned");
    int st = check_stride("new_row_stride", new_row_stride, (int64_t)H_kv * D, eb);
    if (st) return st;
    pkv::AppendFp8Args a{};
    a.k_new = reinterpret_cast<const char*>(k_new);
    a.v_new = reinterpret_cast<const char*>(v_new);
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.positions = positions;
    a.new_row_stride = new_row_stride;
    a.bt_stride = bt_stride;
    a.B = B;
    a.H_kv = H_kv;
    a.n_blocks = n_blocks;
    if (int dc = pkv::debug_check_appends(block_tables, bt_stride, positions, B, block_size, n_blocks, 0, stream))
        return dc;
    hipError_t e = pkv::launch_kv_append_fp8(src_dtype, D, a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append_fp8 launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

int pkv_paged_decode_attention_fp8(int q_dtype, float* out, const void* q, int64_t q_row_stride,
                                   const uint8_t* k_pool, const uint8_t* v_pool, const float* k_scale,
                                   const float* v_scale, const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                   int32_t block_size, int32_t n_blocks, int32_t max_context_len, float scale,
                                   int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    const Fp8Scales sc{k_scale, v_scale, nullptr, nullptr};
    return launch_attention(q_dtype, out, q, q_row_stride, nullptr, nullptr, 0, k_pool, v_pool, nullptr, nullptr,
                            block_tables, bt_stride, context_lens, nullptr, B, H_q, H_kv, D, block_size, n_blocks,
                            max_context_len, scale, partition_size, workspace, workspace_bytes, stream, &sc);
}

int pkv_append_decode_attention_fp8(int q_dtype, float* out, const void* q, int64_t q_row_stride, const void* k_new,
                                    const void* v_new, int64_t new_row_stride, uint8_t* k_pool, uint8_t* v_pool,
                                    float* k_scale, float* v_scale, const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* positions, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                    int32_t block_size, int32_t n_blocks, int32_t max_context_len, float scale,
                                    int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    if (B > 0 && !positions) return fail(PKV_ERR_NULL, "positions is NULL");
    const Fp8Scales sc{k_scale, v_scale, k_scale, v_scale};
    return launch_attention(q_dtype, out, q, q_row_stride, k_new, v_new, new_row_stride, k_pool, v_pool, k_pool,
                            v_pool, block_tables, bt_stride, nullptr, B > 0 ? positions : nullptr, B, H_q, H_kv, D,
                            block_size, n_blocks, max_context_len, scale, partition_size, workspace,
                            workspace_bytes, stream, &sc);
}

int pkv_kv_append_mxfp4(int src_dtype, const void* k_new, const void* v_new, int64_t new_row_stride,
                        uint8_t* k_pool, uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale,
                        const int32_t* block_tables, int32_t bt_stride, const int32_t* positions, int32_t B,
                        int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks, void* stream) {
    const int eb = elem_bytes(src_dtype);
    if (!eb) return fail(PKV_ERR_UNSUPPORTED, "src_dtype %d is not one of PKV_F32/F16/BF16", src_dtype);
    if (B < 0) return fail(PKV_ERR_INVALID_ARG, "B = %d is negative", B);
    if (H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_kv = %d must be positive", H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (bt_stride <= 0) return fail(PKV_ERR_INVALID_ARG, "bt_stride = %d must be positive", bt_stride);
    if (B == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables || !positions)
        return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKV_ERR_INVALID_ARG, "rows and pools must be 16-byte aligned");
    int st = check_stride("new_row_stride", new_row_stride, (int64_t)H_kv * D, eb);
    if (st) return st;
    pkv::AppendMx4Args a{};
    a.k_new = reinterpret_cast<const char*>(k_new);
    a.v_new = reinterpret_cast<const char*>(v_new);
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.positions = positions;
    a.new_row_stride = new_row_stride;
    a.bt_stride = bt_stride;
    a.B = B;
    a.H_kv = H_kv;
    a.n_blocks = n_blocks;
    if (int dc = pkv::debug_check_appends(block_tables, bt_stride, positions, B, block_size, n_blocks, 0, stream))
        return dc;
    hipError_t e = pkv::launch_kv_append_mxfp4(src_dtype, D, a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "kv_append_mxfp4 launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

int pkv_paged_decode_attention_mxfp4(int q_dtype, float* out, const void* q, int64_t q_row_stride,
                                     const uint8_t* k_pool, const uint8_t* v_pool, const uint8_t* k_scale,
                                     const uint8_t* v_scale, const int32_t* block_tables, int32_t bt_stride,
                                     const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                     int32_t block_size, int32_t n_blocks, int32_t max_context_len, float scale,
                                     int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    const Mx4Scales sc{k_scale, v_scale, nullptr, nullptr};
    return launch_attention(q_dtype, out, q, q_row_stride, nullptr, nullptr, 0, k_pool, v_pool, nullptr, nullptr,
                            block_tables, bt_stride, context_lens, nullptr, B, H_q, H_kv, D, block_size, n_blocks,
                            max_context_len, scale, partition_size, workspace, workspace_bytes, stream, nullptr, 0,
                            &sc);
}

int pkv_append_decode_attention_mxfp4(int q_dtype, float* out, const void* q, int64_t q_row_stride,
                                      const void* k_new, const void* v_new, int64_t new_row_stride, uint8_t* k_pool,
                                      uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale,
                                      const int32_t* block_tables, int32_t bt_stride, const int32_t* positions,
                                      int32_t B, int32_t H_q, int32_t H_kv, int32_t D, int32_t block_size,
                                      int32_t n_blocks, int32_t max_context_len, float scale,
                                      int32_t partition_size, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    if (B > 0 && !positions) return fail(PKV_ERR_NULL, "positions is NULL");
    const Mx4Scales sc{k_scale, v_scale, k_scale, v_scale};
    return launch_attention(q_dtype, out, q, q_row_stride, k_new, v_new, new_row_stride, k_pool, v_pool, k_pool,
                            v_pool, block_tables, bt_stride, nullptr, B > 0 ? positions : nullptr, B, H_q, H_kv, D,
                            block_size, n_blocks, max_context_len, scale, partition_size, workspace,
                            workspace_bytes, stream, nullptr, 0, &sc);
}

int pkv_probe_mfma_burn(int32_t n_workgroups, int32_t iterations, void* sink, void* stream) {
    if (!sink) return fail(PKV_ERR_NULL, "sink must not be NULL");
    if (reinterpret_cast<uintptr_t>(sink) & 3u) return fail(PKV_ERR_INVALID_ARG, "sink must be 4-byte aligned");
    if (n_workgroups < 1 || n_workgroups > 65536 || iterations < 1 || iterations > (1 << 30))
        return fail(PKV_ERR_INVALID_ARG, "n_workgroups = %d, iterations = %d", n_workgroups, iterations);
    hipError_t e = pkv::launch_mfma_burn(n_workgroups, iterations, reinterpret_cast<unsigned*>(sink),
                                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return PKV_OK;
}

int pkv_probe_gemm_bf16(int32_t n_workgroups, const void* a, const void* b_t, float* c, int32_t M, int32_t N,
                        int32_t K, void* stream) {
    if (!a || !b_t || !c) return fail(PKV_ERR_NULL, "a, b_t and c must not be NULL");
    if (!aligned16(a) || !aligned16(b_t) || !aligned16(c))
        return fail(PKV_ERR_INVALID_ARG, "a, b_t and c must be 16-byte aligned");
    if (M < 256 || N < 256 || K < 64 || M % 256 || N % 256 || K % 64)
        return fail(PKV_ERR_INVALID_ARG, "M = %d, N = %d (multiples of 256), K = %d (a multiple of 64)", M, N, K);
    if ((int64_t)(M / 256) * (N / 256) > 0x7fffffff || (int64_t)M * K > (1ll << 40) || (int64_t)N * K > (1ll << 40))
        return fail(PKV_ERR_INVALID_ARG, "problem too large");
    if (n_workgroups < 1 || n_workgroups > 65536)
        return fail(PKV_ERR_INVALID_ARG, "n_workgroups = %d is outside [1, 65536]", n_workgroups);
    pkv::GemmArgs g{reinterpret_cast<const char*>(a), reinterpret_cast<const char*>(b_t), c, M, N, K};
    hipError_t e = pkv::launch_gemm_nt_bf16(n_workgroups, g, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return PKV_OK;
}

int pkv_probe_stream_read(const void* buf, size_t bytes, void* sink, int32_t grid, void* stream) {
    if (!buf || !sink) return fail(PKV_ERR_NULL, "buf and sink must not be NULL");
    if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return fail(PKV_ERR_INVALID_ARG, "buf must be 16-byte aligned and sink 4-byte aligned");
    if (bytes < 16 || grid <= 0 || grid > (1 << 20))
        return fail(PKV_ERR_INVALID_ARG, "bytes = %zu, grid = %d", bytes, grid);
    hipError_t e = pkv::launch_stream_read(buf, bytes, reinterpret_cast<unsigned*>(sink), grid,
                                           reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return PKV_OK;
}

int pkv_probe_tile_read(const void* k_pool, const void* v_pool, const void* k_scale, const void* v_scale,
                        int32_t n_blocks, int32_t heads, int32_t tile_bytes, const int32_t* block_ids,
                        int32_t n_items, int32_t team, int32_t paths, int32_t depth, void* sink, int32_t grid,
                        void* stream) {
    if (!k_pool || !v_pool || !block_ids || !sink)
        return fail(PKV_ERR_NULL, "k_pool, v_pool, block_ids and sink must not be NULL");
    if (!k_scale != !v_scale) return fail(PKV_ERR_NULL, "k_scale and v_scale: both or neither");
    if (!aligned16(k_pool) || !aligned16(v_pool) || (reinterpret_cast<uintptr_t>(k_scale) & 3u) ||
        (reinterpret_cast<uintptr_t>(v_scale) & 3u) || (reinterpret_cast<uintptr_t>(block_ids) & 3u) ||
        (reinterpret_cast<uintptr_t>(sink) & 3u))
        return fail(PKV_ERR_INVALID_ARG, "pools must be 16-byte aligned; scales, block_ids and sink 4-byte aligned");
    if (n_blocks <= 0 || heads <= 0 || n_items < 0 || n_items > (1 << 30) || grid <= 0 || grid > 65536)
        return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d, heads = %d, n_items = %d, grid = %d", n_blocks, heads,
                    n_items, grid);
    if (team != 1 && team != 2 && team != 4)
        return fail(PKV_ERR_INVALID_ARG, "team = %d (1, 2 or 4 waves)", team);
    if (heads % team) return fail(PKV_ERR_INVALID_ARG, "heads = %d is not a multiple of team = %d", heads, team);
    if ((paths & 4) && !k_scale) return fail(PKV_ERR_INVALID_ARG, "paths = %d moves scales but there are none", paths);
    if (!pkv::tile_read_variant_exists(tile_bytes, paths, team, depth))
        return fail(PKV_ERR_UNSUPPORTED, "tile_bytes = %d, paths = %d, depth = %d (built: depth 4 with tiles 1024, "
                    "2048, 4096 and paths 0, 1, 5, tiles up to 2048 also 7, 1024 also 4, 6; depths 2 and 8 with "
                    "tiles 1024 and paths 0, 4, 6, 7)", tile_bytes, paths, depth);
    if (n_items == 0) {
        g_err[0] = 0;
        return PKV_OK;
    }
    pkv::TileReadArgs a{};
    a.k_pool = static_cast<const char*>(k_pool);
    a.v_pool = static_cast<const char*>(v_pool);
    a.k_scale = static_cast<const char*>(k_scale);
    a.v_scale = static_cast<const char*>(v_scale);
    a.ids = block_ids;
    a.sink = reinterpret_cast<unsigned*>(sink);
    a.n_blocks = n_blocks;
    a.heads = heads;
    a.n_items = n_items;
    a.scales = k_scale != nullptr;
    hipError_t e = pkv::launch_tile_read(a, tile_bytes, paths, team, depth, grid,
                                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
    g_err[0] = 0;
    return PKV_OK;
}

int pkv_copy_blocks(int dtype, void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst, int32_t n,
                    int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks, void* stream) {
    const int eb = elem_bytes(dtype);
    if (!eb) return fail(PKV_ERR_UNSUPPORTED, "dtype %d is not one of PKV_F32/F16/BF16", dtype);
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n = %d is negative", n);
    if (H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_kv = %d must be positive", H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (n == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!k_pool || !v_pool || !src || !dst) return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(k_pool) || !aligned16(v_pool))
        return fail(PKV_ERR_INVALID_ARG, "the pools must be 16-byte aligned");
    pkv::CopyArgs a{};
    a.k_pool = reinterpret_cast<char*>(k_pool);
    a.v_pool = reinterpret_cast<char*>(v_pool);
    a.src = src;
    a.dst = dst;
    a.n = n;
    a.n_blocks = n_blocks;
    a.block_bytes = (int64_t)H_kv * block_size * D * eb;
    if ((int64_t)n * 2 * ((a.block_bytes + pkv::kCopyPieceBytes - 1) / pkv::kCopyPieceBytes) > 0x7fffffff)
        return fail(PKV_ERR_INVALID_ARG, "grid too large");
    hipError_t e = pkv::launch_copy_blocks(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

int pkv_copy_blocks_fp8(uint8_t* k_pool, uint8_t* v_pool, float* k_scale, float* v_scale, const int32_t* src,
                        const int32_t* dst, int32_t n, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                        void* stream) {
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n = %d is negative", n);
    if (H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_kv = %d must be positive", H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (n == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!k_pool || !v_pool || !k_scale || !v_scale || !src || !dst) return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_scale) || !aligned16(v_scale))
        return fail(PKV_ERR_INVALID_ARG, "pools and scale arrays must be 16-byte aligned");
    pkv::CopyArgs a{};
    a.src = src;
    a.dst = dst;
    a.n = n;
    a.n_blocks = n_blocks;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // codes: H_kv * block_size * D bytes per block; scales: H_kv * block_size floats per block
    a.k_pool = reinterpret_cast<char*>(k_pool);
    a.v_pool = reinterpret_cast<char*>(v_pool);
    a.block_bytes = (int64_t)H_kv * block_size * D;
    hipError_t e = pkv::launch_copy_blocks(a, s);
    if (e == hipSuccess) {
        a.k_pool = reinterpret_cast<char*>(k_scale);
        a.v_pool = reinterpret_cast<char*>(v_scale);
        a.block_bytes = (int64_t)H_kv * block_size * 4;
        e = pkv::launch_copy_blocks(a, s);
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "copy_blocks_fp8 launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

int pkv_copy_blocks_mxfp4(uint8_t* k_pool, uint8_t* v_pool, uint8_t* k_scale, uint8_t* v_scale, const int32_t* src,
                          const int32_t* dst, int32_t n, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                          void* stream) {
    if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n = %d is negative", n);
    if (H_kv <= 0) return fail(PKV_ERR_INVALID_ARG, "H_kv = %d must be positive", H_kv);
    if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head dim D = %d (built: 64, 128)", D);
    if (block_size != pkv::kBlockSize)
        return fail(PKV_ERR_UNSUPPORTED, "block_size = %d (built: %d)", block_size, pkv::kBlockSize);
    if (n_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "n_blocks = %d must be positive", n_blocks);
    if (n == 0) {
        pkv::clear_error();
        return PKV_OK;
    }
    if (!k_pool || !v_pool || !k_scale || !v_scale || !src || !dst) return fail(PKV_ERR_NULL, "a required pointer is NULL");
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_scale) || !aligned16(v_scale))
        return fail(PKV_ERR_INVALID_ARG, "pools and scale arrays must be 16-byte aligned");
    pkv::CopyArgs a{};
    a.src = src;
    a.dst = dst;
    a.n = n;
    a.n_blocks = n_blocks;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // codes: H_kv * block_size * D/2 bytes per block; scales: H_kv * block_size * D/32 bytes per
    // block (both multiples of the copy's 16-byte grain)
    a.k_pool = reinterpret_cast<char*>(k_pool);
    a.v_pool = reinterpret_cast<char*>(v_pool);
    a.block_bytes = (int64_t)H_kv * block_size * (D / 2);
    hipError_t e = pkv::launch_copy_blocks(a, s);
    if (e == hipSuccess) {
        a.k_pool = reinterpret_cast<char*>(k_scale);
        a.v_pool = reinterpret_cast<char*>(v_scale);
        a.block_bytes = (int64_t)H_kv * block_size * (D / 32);
        e = pkv::launch_copy_blocks(a, s);
    }
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "copy_blocks_mxfp4 launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

size_t pkv_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t D, int32_t max_context_len,
                                  int32_t partition_size) {
    if (B <= 0 || H_q <= 0 || D <= 0 || max_context_len <= 0 || partition_size <= 0) return 0;
    // the KV-head count and dtype do not change the workspace
    const Plan p = make_plan(PKV_F16, B, H_q, H_q, D, max_context_len, partition_size);
    return p.ws_total;
}

int pkv_paged_decode_attention(int dtype, float* out, const void* q, int64_t q_row_stride, const void* k_pool,
                               const void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                               const int32_t* context_lens, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                               int32_t block_size, int32_t n_blocks, int32_t max_context_len, float scale,
                               int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
    return launch_attention(dtype, out, q, q_row_stride, nullptr, nullptr, 0, k_pool, v_pool, nullptr, nullptr,
                            block_tables, bt_stride, context_lens, nullptr, B, H_q, H_kv, D, block_size, n_blocks,
                            max_context_len, scale, partition_size, workspace, workspace_bytes, stream);
}

int pkv_append_decode_attention(int dtype, float* out, const void* q, int64_t q_row_stride, const void* k_new,
                                const void* v_new, int64_t new_row_stride, void* k_pool, void* v_pool,
                                const int32_t* block_tables, int32_t bt_stride, const int32_t* positions, int32_t B,
                                int32_t H_q, int32_t H_kv, int32_t D, int32_t block_size, int32_t n_blocks,
                                int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (B > 0 && !positions) return fail(PKV_ERR_NULL, "positions is NULL");
    return launch_attention(dtype, out, q, q_row_stride, k_new, v_new, new_row_stride, k_pool, v_pool, k_pool, v_pool,
                            block_tables, bt_stride, nullptr, B > 0 ? positions : nullptr, B, H_q, H_kv, D,
                            block_size, n_blocks, max_context_len, scale, partition_size, workspace,
                            workspace_bytes, stream);
}

int pkv_append_decode_attention_persistent(int dtype, float* out, const void* q, int64_t q_row_stride,
                                           const void* k_new, const void* v_new, int64_t new_row_stride, void* k_pool,
                                           void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                                           const int32_t* positions, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                           int32_t block_size, int32_t n_blocks, int32_t max_context_len, float scale,
                                           int32_t partition_size, void* workspace, size_t workspace_bytes,
                                           int32_t n_workgroups, void* stream) {
    if (n_workgroups < 1 || n_workgroups > 65536)
        return fail(PKV_ERR_INVALID_ARG, "n_workgroups = %d is outside [1, 65536]", n_workgroups);
    if (B > 0 && !positions) return fail(PKV_ERR_NULL, "positions is NULL");
    return launch_attention(dtype, out, q, q_row_stride, k_new, v_new, new_row_stride, k_pool, v_pool, k_pool, v_pool,
                            block_tables, bt_stride, nullptr, B > 0 ? positions : nullptr, B, H_q, H_kv, D,
                            block_size, n_blocks, max_context_len, scale, partition_size, workspace,
                            workspace_bytes, stream, nullptr, n_workgroups);
}

int pkv_append_decode_attention_noalloc(int dtype, float* out, const void* q, int64_t q_row_stride,
                                        const void* k_new, const void* v_new, int64_t new_row_stride, void* k_pool,
                                        void* v_pool, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* positions, int32_t B, int32_t H_q, int32_t H_kv, int32_t D,
                                        int32_t block_size, int32_t n_blocks, int32_t max_context_len, float scale,
                                        int32_t partition_size, void* stream) {
    const size_t need = pkv_decode_workspace_bytes(B, H_q, D, max_context_len, partition_size);
    if (need > kScratchBytes)
        return fail(PKV_ERR_WORKSPACE,
                    "the split needs %zu bytes of partials; the allocation-free step holds at most %zu "
                    "(use pkv_append_decode_attention with a workspace, or a larger partition_size)",
                    need, kScratchBytes);
    void* ws = nullptr;
    if (need) {
        const int st = scratch_for_current_device(&ws);
        if (st) return st;
    }
    return pkv_append_decode_attention(dtype, out, q, q_row_stride, k_new, v_new, new_row_stride, k_pool, v_pool,
                                       block_tables, bt_stride, positions, B, H_q, H_kv, D, block_size, n_blocks,
                                       max_context_len, scale, partition_size, ws, need ? kScratchBytes : 0, stream);
}

}  // extern "C"
