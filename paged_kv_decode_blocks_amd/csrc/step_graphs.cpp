// step_graphs.cpp -- the decode step captured as HIP graphs over a grid of
// (batch capacity, context capacity) buckets (C ABI in include/pkv.h).
//
// A small decode batch runs its kernels in tens of microseconds, less than the
// host needs to launch them one by one ("Injecting Adrenaline into LLM
// Serving" review, section 3.2.2, on graphs captured over a two-dimensional
// capacity grid and the smallest fitting one replayed).  Every bucket's graph
// is the same stream-ordered sequence the eager calls enqueue -- block copies
// for copy-on-write, then the fused append + attention (+ the split merge) --
// captured once over the caller's fixed buffers.  Replaying costs one
// hipGraphLaunch.  The capture uses the library's own entry points, so the
// graphs run exactly the kernels and launch shapes of the eager path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "pkv.h"
#include "pkv_host.h"

using pkv::fail;

struct pkv_step_graphs {
    pkv_step_desc desc;
    std::vector<int32_t> bcaps, ccaps;
    int variants;                            // 1: no copy node; 2: also a variant with the copy node
    std::vector<hipGraph_t> graphs;          // [(i_b * n_ctx + i_c) * variants + with_copy]
    std::vector<hipGraphExec_t> execs;

    ~pkv_step_graphs() {
        for (hipGraphExec_t e : execs)
            if (e) (void)hipGraphExecDestroy(e);
        for (hipGraph_t g : graphs)
            if (g) (void)hipGraphDestroy(g);
    }
};

namespace {

bool strictly_increasing_positive(const int32_t* v, int32_t n) {
    for (int32_t i = 0; i < n; ++i)
        if (v[i] <= 0 || (i && v[i] <= v[i - 1])) return false;
    return true;
}

// Enqueue one bucket's step on `s` (capturing).  Returns a pkv_status.
int enqueue_step(const pkv_step_desc& d, int32_t Bc, int32_t Cc, bool with_copy, hipStream_t s) {
    const bool fp8 = d.k_scale != nullptr;
    const bool mx4 = d.k_mx_scale != nullptr;
    uint8_t* kp = static_cast<uint8_t*>(d.k_pool);
    uint8_t* vp = static_cast<uint8_t*>(d.v_pool);
    if (with_copy) {
        const int st = fp8   ? pkv_copy_blocks_fp8(kp, vp, d.k_scale, d.v_scale, d.cow_src, d.cow_dst, Bc, d.H_kv,
                                                   d.D, d.block_size, d.n_blocks, s)
                       : mx4 ? pkv_copy_blocks_mxfp4(kp, vp, d.k_mx_scale, d.v_mx_scale, d.cow_src, d.cow_dst, Bc,
                                                     d.H_kv, d.D, d.block_size, d.n_blocks, s)
                             : pkv_copy_blocks(d.dtype, d.k_pool, d.v_pool, d.cow_src, d.cow_dst, Bc, d.H_kv, d.D,
                                               d.block_size, d.n_blocks, s);
        if (st) return st;
    }
    if (mx4)
        return pkv_append_decode_attention_mxfp4(d.dtype, d.out, d.q, d.q_row_stride, d.k_new, d.v_new,
                                                 d.new_row_stride, kp, vp, d.k_mx_scale, d.v_mx_scale,
                                                 d.block_tables, d.bt_stride, d.positions, Bc, d.H_q, d.H_kv, d.D,
                                                 d.block_size, d.n_blocks, Cc, d.scale, d.partition_size,
                                                 d.workspace, d.workspace_bytes, s);
    if (fp8)
        return pkv_append_decode_attention_fp8(d.dtype, d.out, d.q, d.q_row_stride, d.k_new, d.v_new,
                                               d.new_row_stride, static_cast<uint8_t*>(d.k_pool),
                                               static_cast<uint8_t*>(d.v_pool), d.k_scale, d.v_scale,
                                               d.block_tables, d.bt_stride, d.positions, Bc, d.H_q, d.H_kv, d.D,
                                               d.block_size, d.n_blocks, Cc, d.scale, d.partition_size,
                                               d.workspace, d.workspace_bytes, s);
    return pkv_append_decode_attention(d.dtype, d.out, d.q, d.q_row_stride, d.k_new, d.v_new, d.new_row_stride,
                                       d.k_pool, d.v_pool, d.block_tables, d.bt_stride, d.positions, Bc, d.H_q,
                                       d.H_kv, d.D, d.block_size, d.n_blocks, Cc, d.scale, d.partition_size,
                                       d.workspace, d.workspace_bytes, s);
}

}  // namespace

extern "C" {

pkv_step_graphs* pkv_step_graphs_create(const pkv_step_desc* desc, const int32_t* batch_caps, int32_t n_batch,
                                        const int32_t* ctx_caps, int32_t n_ctx) {
    if (!desc || !batch_caps || !ctx_caps) {
        fail(PKV_ERR_NULL, "desc, batch_caps and ctx_caps must not be NULL");
        return nullptr;
    }
    if (n_batch <= 0 || n_ctx <= 0 || n_batch > 4096 || n_ctx > 4096) {
        fail(PKV_ERR_INVALID_ARG, "n_batch = %d and n_ctx = %d must lie in [1, 4096]", n_batch, n_ctx);
        return nullptr;
    }
    if (!strictly_increasing_positive(batch_caps, n_batch) || !strictly_increasing_positive(ctx_caps, n_ctx)) {
        fail(PKV_ERR_INVALID_ARG, "capacity lists must be positive and strictly increasing");
        return nullptr;
    }
    if (!desc->positions || !desc->block_tables) {
        fail(PKV_ERR_NULL, "positions and block_tables must not be NULL");
        return nullptr;
    }
    if (!desc->cow_src != !desc->cow_dst) {
        fail(PKV_ERR_INVALID_ARG, "cow_src and cow_dst must both be set or both be NULL");
        return nullptr;
    }
    if (!desc->k_scale != !desc->v_scale || !desc->k_mx_scale != !desc->v_mx_scale ||
        (desc->k_scale && desc->k_mx_scale)) {
        fail(PKV_ERR_INVALID_ARG, "set k_scale and v_scale (FP8 pools) or k_mx_scale and v_mx_scale (MXFP4 pools), "
             "both of a pair or neither");
        return nullptr;
    }
    const int32_t maxB = batch_caps[n_batch - 1], maxC = ctx_caps[n_ctx - 1];
    if ((int64_t)maxC > (int64_t)desc->bt_stride * desc->block_size) {
        fail(PKV_ERR_INVALID_ARG, "largest context capacity %d exceeds bt_stride * block_size = %lld", maxC,
             (long long)desc->bt_stride * desc->block_size);
        return nullptr;
    }
    if (desc->partition_size > 0) {
        const size_t need = pkv_decode_workspace_bytes(maxB, desc->H_q, desc->D, maxC, desc->partition_size);
        if (desc->workspace_bytes < need || (need && !desc->workspace)) {
            fail(PKV_ERR_WORKSPACE, "the largest bucket needs %zu bytes of workspace, got %zu", need,
                 desc->workspace_bytes);
            return nullptr;
        }
    }
    pkv_step_graphs* g = new (std::nothrow) pkv_step_graphs();
    if (!g) {
        fail(PKV_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    g->desc = *desc;
    g->bcaps.assign(batch_caps, batch_caps + n_batch);
    g->ccaps.assign(ctx_caps, ctx_caps + n_ctx);
    g->variants = desc->cow_src ? 2 : 1;
    g->graphs.assign((size_t)n_batch * n_ctx * g->variants, nullptr);
    g->execs.assign((size_t)n_batch * n_ctx * g->variants, nullptr);

    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) {
        fail(PKV_ERR_HIP, "capture stream: %s", hipGetErrorString(e));
        delete g;
        return nullptr;
    }
    int status = PKV_OK;
    const size_t n_graphs = g->graphs.size();
    for (size_t k = 0; k < n_graphs && status == PKV_OK; ++k) {
        {
            const bool with_copy = k % g->variants == 1;
            const size_t bucket = k / g->variants;
            const int32_t ib = (int32_t)(bucket / n_ctx), ic = (int32_t)(bucket % n_ctx);
            e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
            if (e != hipSuccess) {
                status = fail(PKV_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
                break;
            }
            const int st = enqueue_step(g->desc, g->bcaps[ib], g->ccaps[ic], with_copy, cs);
            hipGraph_t graph = nullptr;
            e = hipStreamEndCapture(cs, &graph);
            if (st != PKV_OK) {
                if (graph) (void)hipGraphDestroy(graph);
                status = st;   // pkv_last_error() already holds the detail
                break;
            }
            if (e != hipSuccess || !graph) {
                if (graph) (void)hipGraphDestroy(graph);
                status = fail(PKV_ERR_HIP, "end capture: %s", hipGetErrorString(e));
                break;
            }
            g->graphs[k] = graph;
            e = hipGraphInstantiate(&g->execs[k], graph, nullptr, nullptr, 0);
            if (e != hipSuccess) {
                g->execs[k] = nullptr;
                status = fail(PKV_ERR_HIP, "instantiate: %s", hipGetErrorString(e));
            }
        }
    }
    (void)hipStreamDestroy(cs);
    if (status != PKV_OK) {
        delete g;
        return nullptr;
    }
    pkv::clear_error();
    return g;
}

int pkv_step_graphs_launch(pkv_step_graphs* g, int32_t B, int32_t max_context_len, int32_t n_copies, void* stream) {
    if (!g) return fail(PKV_ERR_NULL, "step graphs object is NULL");
    if (B < 0 || max_context_len < 0 || n_copies < 0)
        return fail(PKV_ERR_INVALID_ARG, "B = %d, max_context_len = %d, n_copies = %d", B, max_context_len, n_copies);
    if (n_copies > 0 && g->variants == 1)
        return fail(PKV_ERR_INVALID_ARG, "n_copies = %d but the graphs were captured without copy buffers", n_copies);
    auto ib = std::lower_bound(g->bcaps.begin(), g->bcaps.end(), std::max(B, 1));
    auto ic = std::lower_bound(g->ccaps.begin(), g->ccaps.end(), std::max(max_context_len, 1));
    if (ib == g->bcaps.end())
        return fail(PKV_ERR_INVALID_ARG, "B = %d exceeds the largest batch capacity %d", B, g->bcaps.back());
    if (ic == g->ccaps.end())
        return fail(PKV_ERR_INVALID_ARG, "max_context_len = %d exceeds the largest context capacity %d",
                    max_context_len, g->ccaps.back());
    if (n_copies > *ib)
        return fail(PKV_ERR_INVALID_ARG, "n_copies = %d exceeds the batch capacity %d", n_copies, *ib);
    const size_t bucket = (size_t)(ib - g->bcaps.begin()) * g->ccaps.size() + (size_t)(ic - g->ccaps.begin());
    const size_t k = bucket * g->variants + (n_copies > 0 ? 1 : 0);
    const hipError_t e = hipGraphLaunch(g->execs[k], reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

void pkv_step_graphs_destroy(pkv_step_graphs* g) { delete g; }

}  // extern "C"

// ---------------------------------------------------------------------------
// Two attention batches per step, captured over a (local capacity, offloaded
// capacity) grid.  The Adrenaline review (section 3.2.1) runs the decode
// instance's own attention and the attention it offloaded to another GPU at the
// same time, and (section 3.2.2) captures graphs over both batch sizes; on one
// GPU the two batches are two step descriptions with their own tables, pools and
// workspaces, captured as two parallel branches of one graph (or one after the
// other, to measure what the overlap buys).
// ---------------------------------------------------------------------------
struct pkv_dual_step_graphs {
    pkv_step_desc desc[2];
    std::vector<int32_t> caps[2];
    int32_t ctx_cap = 0;
    std::vector<hipGraph_t> graphs;          // [i_local * n_off + i_off]; the (0, 0) bucket has none
    std::vector<hipGraphExec_t> execs;

    ~pkv_dual_step_graphs() {
        for (hipGraphExec_t e : execs)
            if (e) (void)hipGraphExecDestroy(e);
        for (hipGraph_t g : graphs)
            if (g) (void)hipGraphDestroy(g);
    }
};

namespace {

bool increasing_from_zero(const int32_t* v, int32_t n) {
    for (int32_t i = 0; i < n; ++i)
        if (v[i] < 0 || (i && v[i] <= v[i - 1])) return false;
    return true;
}

int check_branch(const pkv_step_desc* d, const char* name, int32_t max_cap, int32_t ctx_cap) {
    if (!d->positions || !d->block_tables) return fail(PKV_ERR_NULL, "%s: positions and block_tables must be set", name);
    if (d->cow_src || d->cow_dst) return fail(PKV_ERR_UNSUPPORTED, "%s: no copy-on-write node in a dual step", name);
    if (!d->k_scale != !d->v_scale || !d->k_mx_scale != !d->v_mx_scale || (d->k_scale && d->k_mx_scale))
        return fail(PKV_ERR_INVALID_ARG, "%s: set one pair of scale pools at most, both of a pair", name);
    if ((int64_t)ctx_cap > (int64_t)d->bt_stride * d->block_size)
        return fail(PKV_ERR_INVALID_ARG, "%s: context capacity %d exceeds bt_stride * block_size", name, ctx_cap);
    if (d->partition_size > 0 && max_cap > 0) {
        const size_t need = pkv_decode_workspace_bytes(max_cap, d->H_q, d->D, ctx_cap, d->partition_size);
        if (d->workspace_bytes < need || (need && !d->workspace))
            return fail(PKV_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got %zu", name, need, d->workspace_bytes);
    }
    return PKV_OK;
}

}  // namespace

extern "C" {

pkv_dual_step_graphs* pkv_dual_step_graphs_create(const pkv_step_desc* local, const pkv_step_desc* offloaded,
                                                  const int32_t* local_caps, int32_t n_local,
                                                  const int32_t* off_caps, int32_t n_off, int32_t ctx_cap,
                                                  int parallel) {
    if (!local || !offloaded || !local_caps || !off_caps) {
        fail(PKV_ERR_NULL, "descriptions and capacity lists must not be NULL");
        return nullptr;
    }
    if (n_local <= 0 || n_off <= 0 || n_local > 1024 || n_off > 1024 || ctx_cap <= 0) {
        fail(PKV_ERR_INVALID_ARG, "n_local = %d, n_off = %d in [1, 1024]; ctx_cap = %d > 0", n_local, n_off, ctx_cap);
        return nullptr;
    }
    if (!increasing_from_zero(local_caps, n_local) || !increasing_from_zero(off_caps, n_off)) {
        fail(PKV_ERR_INVALID_ARG, "capacity lists must be non-negative and strictly increasing");
        return nullptr;
    }
    if (check_branch(local, "local", local_caps[n_local - 1], ctx_cap) ||
        check_branch(offloaded, "offloaded", off_caps[n_off - 1], ctx_cap))
        return nullptr;
    if (local->partition_size > 0 && offloaded->partition_size > 0 && local->workspace &&
        local->workspace == offloaded->workspace) {
        fail(PKV_ERR_WORKSPACE, "the two branches run at the same time: give each its own workspace");
        return nullptr;
    }
    pkv_dual_step_graphs* g = new (std::nothrow) pkv_dual_step_graphs();
    if (!g) {
        fail(PKV_ERR_INVALID_ARG, "out of host memory");
        return nullptr;
    }
    g->desc[0] = *local;
    g->desc[1] = *offloaded;
    g->caps[0].assign(local_caps, local_caps + n_local);
    g->caps[1].assign(off_caps, off_caps + n_off);
    g->ctx_cap = ctx_cap;
    const size_t n = (size_t)n_local * n_off;
    g->graphs.assign(n, nullptr);
    g->execs.assign(n, nullptr);

    hipStream_t s0 = nullptr, s1 = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s0, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&s1, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join, hipEventDisableTiming);
    int status = e == hipSuccess ? PKV_OK : fail(PKV_ERR_HIP, "capture streams: %s", hipGetErrorString(e));
    for (size_t k = 0; k < n && status == PKV_OK; ++k) {
        const int32_t c0 = g->caps[0][k / n_off], c1 = g->caps[1][k % n_off];
        if (c0 == 0 && c1 == 0) continue;   // nothing to run
        e = hipStreamBeginCapture(s0, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) {
            status = fail(PKV_ERR_HIP, "begin capture: %s", hipGetErrorString(e));
            break;
        }
        int st = PKV_OK;
        const bool both = c0 > 0 && c1 > 0;
        hipStream_t s_off = both && parallel ? s1 : s0;
        if (both && parallel) {   // fork: s1 joins the capture after this point of s0
            e = hipEventRecord(fork, s0);
            if (e == hipSuccess) e = hipStreamWaitEvent(s1, fork, 0);
            if (e != hipSuccess) st = fail(PKV_ERR_HIP, "fork: %s", hipGetErrorString(e));
        }
        if (st == PKV_OK && c0 > 0) st = enqueue_step(g->desc[0], c0, ctx_cap, false, s0);
        if (st == PKV_OK && c1 > 0) st = enqueue_step(g->desc[1], c1, ctx_cap, false, s_off);
        if (st == PKV_OK && both && parallel) {   // join the offloaded branch back into s0
            e = hipEventRecord(join, s1);
            if (e == hipSuccess) e = hipStreamWaitEvent(s0, join, 0);
            if (e != hipSuccess) st = fail(PKV_ERR_HIP, "join: %s", hipGetErrorString(e));
        }
        hipGraph_t graph = nullptr;
        e = hipStreamEndCapture(s0, &graph);
        if (st != PKV_OK || e != hipSuccess || !graph) {
            if (graph) (void)hipGraphDestroy(graph);
            status = st != PKV_OK ? st : fail(PKV_ERR_HIP, "end capture: %s", hipGetErrorString(e));
            break;
        }
        g->graphs[k] = graph;
        e = hipGraphInstantiate(&g->execs[k], graph, nullptr, nullptr, 0);
        if (e != hipSuccess) {
            g->execs[k] = nullptr;
            status = fail(PKV_ERR_HIP, "instantiate: %s", hipGetErrorString(e));
        }
    }
    if (join) (void)hipEventDestroy(join);
    if (fork) (void)hipEventDestroy(fork);
    if (s1) (void)hipStreamDestroy(s1);
    if (s0) (void)hipStreamDestroy(s0);
    if (status != PKV_OK) {
        delete g;
        return nullptr;
    }
    pkv::clear_error();
    return g;
}

int pkv_dual_step_graphs_launch(pkv_dual_step_graphs* g, int32_t B_local, int32_t B_off, void* stream) {
    if (!g) return fail(PKV_ERR_NULL, "dual step graphs object is NULL");
    if (B_local < 0 || B_off < 0) return fail(PKV_ERR_INVALID_ARG, "B_local = %d, B_off = %d", B_local, B_off);
    auto i0 = std::lower_bound(g->caps[0].begin(), g->caps[0].end(), B_local);
    auto i1 = std::lower_bound(g->caps[1].begin(), g->caps[1].end(), B_off);
    if (i0 == g->caps[0].end() || i1 == g->caps[1].end())
        return fail(PKV_ERR_INVALID_ARG, "B_local = %d / B_off = %d exceed the largest capacities %d / %d", B_local,
                    B_off, g->caps[0].back(), g->caps[1].back());
    const size_t k = (size_t)(i0 - g->caps[0].begin()) * g->caps[1].size() + (size_t)(i1 - g->caps[1].begin());
    if (!g->execs[k]) {   // both capacities 0: an empty step
        pkv::clear_error();
        return PKV_OK;
    }
    const hipError_t e = hipGraphLaunch(g->execs[k], reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "graph launch: %s", hipGetErrorString(e));
    pkv::clear_error();
    return PKV_OK;
}

void pkv_dual_step_graphs_destroy(pkv_dual_step_graphs* g) { delete g; }

}  // extern "C"
