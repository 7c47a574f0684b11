// pkv_cumask.cpp -- decode attention on CU-limited streams, as a standalone
// program (built next to libpkv.so; uses the library's C ABI and rocBLAS).
//
// Decode attention is memory-bound, so a fraction of the GPU's compute units
// already draws most of the HBM bandwidth and the rest can run other work
// ("Injecting Adrenaline into LLM Serving" review, section 3.3).  This program
// measures that on MI355X with CU-masked streams.  It is a separate process on
// purpose: a process that has loaded PyTorch runs PyTorch's bundled HIP
// runtime, whose CU-masked queue creation fails on this system; here the
// library and rocBLAS run on the system ROCm runtime.
//
//   pkv_cumask check DIR
//       Reads a decode step from DIR (meta.txt and raw .bin arrays), runs it on
//       the default stream and on CU-masked streams (8 spread, 32 first, 128
//       spread), each from fresh copies of the inputs, and writes the outputs
//       and the pools after the step to DIR/out_<tag>.bin, DIR/k_pool_<tag>.bin,
//       DIR/v_pool_<tag>.bin.
//
//   pkv_cumask sweep dtype B H_q H_kv D P append pool_factor seed steps len0,len1,...
//       Synthetic step of that shape (context lengths as given, blocks scattered
//       over a pool pool_factor times the blocks needed, K/V and q filled with
//       seeded finite values), resident in HBM and rotated over enough copies
//       to defeat the 256 MB Infinity Cache.  Prints one JSON object: step
//       bandwidth on 8 .. all CUs (spread over the CU numbering or packed at
//       its start), then the step on a spread subset beside a bf16 8192^3
//       rocBLAS GEMM looping on the complementary CUs, each also alone on its
//       subset, and both sharing the whole GPU.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "pkv.h"

namespace {

#define CHECK_HIP(x)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            exit(2);                                                                          \
        }                                                                                     \
    } while (0)
#define CHECK_PKV(x)                                                                                     \
    do {                                                                                                 \
        int s_ = (x);                                                                                    \
        if (s_ != PKV_OK) {                                                                              \
            fprintf(stderr, "%s:%d %s: %s: %s\n", __FILE__, __LINE__, #x, pkv_status_string(s_), pkv_last_error()); \
            exit(3);                                                                                     \
        }                                                                                                \
    } while (0)

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Seeded finite values: 16-bit elements with a fixed small exponent and random
// sign and mantissa (|x| in [0.25, 0.5) for f16 and bf16); f32 the same magnitude.
__global__ void fill_kernel(uint16_t* p, size_t n, uint64_t seed, int bf16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) {
        uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
        z = (z ^ (z >> 31)) * 0xBF58476D1CE4E5B9ull;
        z ^= z >> 29;
        const uint16_t r = (uint16_t)z;
        p[i] = bf16 ? (uint16_t)((r & 0x807F) | 0x3E80) : (uint16_t)((r & 0x83FF) | 0x3400);
    }
}

void fill(void* p, size_t bytes, uint64_t seed, int dtype) {
    hipLaunchKernelGGL(fill_kernel, dim3(4096), dim3(256), 0, nullptr, (uint16_t*)p, bytes / 2, seed,
                       dtype == PKV_BF16 ? 1 : 0);
    CHECK_HIP(hipGetLastError());
}

int elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : 2; }

// One decode step's device buffers and its launch.
struct Step {
    int dtype = PKV_F16, B = 0, H_q = 0, H_kv = 0, D = 0, n_blocks = 0, W = 0, P = 0, max_ctx = 0;
    bool append = true;
    float scale = 1.0f;
    void *q = nullptr, *k_pool = nullptr, *v_pool = nullptr, *k_new = nullptr, *v_new = nullptr;
    int32_t *bt = nullptr, *pos = nullptr, *ctx = nullptr;
    float* out = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    size_t pool_bytes() const { return (size_t)n_blocks * H_kv * 16 * D * elem_bytes(dtype); }

    void alloc() {
        const int e = elem_bytes(dtype);
        CHECK_HIP(hipMalloc(&q, (size_t)B * H_q * D * e));
        CHECK_HIP(hipMalloc(&k_pool, pool_bytes()));
        CHECK_HIP(hipMalloc(&v_pool, pool_bytes()));
        CHECK_HIP(hipMalloc(&k_new, (size_t)B * H_kv * D * e));
        CHECK_HIP(hipMalloc(&v_new, (size_t)B * H_kv * D * e));
        CHECK_HIP(hipMalloc((void**)&bt, (size_t)B * W * 4));
        CHECK_HIP(hipMalloc((void**)&pos, (size_t)B * 4));
        CHECK_HIP(hipMalloc((void**)&ctx, (size_t)B * 4));
        CHECK_HIP(hipMalloc((void**)&out, (size_t)B * H_q * D * 4));
        ws_bytes = P ? pkv_decode_workspace_bytes(B, H_q, D, max_ctx, P) : 0;
        if (ws_bytes) CHECK_HIP(hipMalloc(&ws, ws_bytes));
    }
    void release() {
        for (void* p : {q, k_pool, v_pool, k_new, v_new, (void*)bt, (void*)pos, (void*)ctx, (void*)out, ws})
            if (p) CHECK_HIP(hipFree(p));
    }
    int launch(hipStream_t s) const {
        if (append)
            return pkv_append_decode_attention(dtype, out, q, (int64_t)H_q * D, k_new, v_new, (int64_t)H_kv * D,
                                               k_pool, v_pool, bt, W, pos, B, H_q, H_kv, D, 16, n_blocks, max_ctx,
                                               scale, P, ws, ws_bytes, s);
        return pkv_paged_decode_attention(dtype, out, q, (int64_t)H_q * D, k_pool, v_pool, bt, W, ctx, B, H_q, H_kv,
                                          D, 16, n_blocks, max_ctx, scale, P, ws, ws_bytes, s);
    }
};

std::vector<char> read_file(const std::string& path) {
    FILE* f = fopen(path.c_str(), "rb");
    if (!f) {
        fprintf(stderr, "cannot open %s\n", path.c_str());
        exit(4);
    }
    fseek(f, 0, SEEK_END);
    const long n = ftell(f);
    fseek(f, 0, SEEK_SET);
    std::vector<char> v((size_t)n);
    if (n && fread(v.data(), 1, (size_t)n, f) != (size_t)n) exit(4);
    fclose(f);
    return v;
}

void write_file(const std::string& path, const void* p, size_t n) {
    FILE* f = fopen(path.c_str(), "wb");
    if (!f || fwrite(p, 1, n, f) != n) {
        fprintf(stderr, "cannot write %s\n", path.c_str());
        exit(4);
    }
    fclose(f);
}

void upload(void* dst, const std::string& path, size_t expect) {
    const std::vector<char> v = read_file(path);
    if (v.size() != expect) {
        fprintf(stderr, "%s: %zu bytes, expected %zu\n", path.c_str(), v.size(), expect);
        exit(4);
    }
    CHECK_HIP(hipMemcpy(dst, v.data(), expect, hipMemcpyHostToDevice));
}

hipStream_t masked_stream(int n_cus, int count, int layout) {
    std::vector<uint32_t> mask((n_cus + 31) / 32);
    CHECK_PKV(pkv_cu_mask(n_cus, count, layout, mask.data(), (int32_t)mask.size()));
    fprintf(stderr, "pkv_cumask: creating a stream on %d of %d CUs (%s)\n", count, n_cus, layout ? "spread" : "first");
    void* s = nullptr;
    CHECK_PKV(pkv_stream_create_cu_masked(mask.data(), (int32_t)mask.size(), &s));
    fprintf(stderr, "pkv_cumask: stream created\n");
    return (hipStream_t)s;
}

int run_check(const std::string& dir) {
    Step st;
    {
        FILE* f = fopen((dir + "/meta.txt").c_str(), "r");
        int app = 0;
        if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %d %d %f", &st.dtype, &st.B, &st.H_q, &st.H_kv, &st.D,
                         &st.n_blocks, &st.W, &st.P, &st.max_ctx, &app, &st.scale) != 11) {
            fprintf(stderr, "bad meta.txt\n");
            return 4;
        }
        fclose(f);
        st.append = app != 0;
    }
    fprintf(stderr, "pkv_cumask: allocating\n");
    st.alloc();
    const int e = elem_bytes(st.dtype);
    const int n_cus = pkv_device_cu_count();
    fprintf(stderr, "pkv_cumask: %d CUs\n", n_cus);
    struct Run { const char* tag; int count, layout; };
    const Run runs[] = {{"full", 0, 0}, {"m8_spread", 8, 1}, {"m32_first", 32, 0}, {"m128_spread", 128, 1}};
    for (const Run& r : runs) {
        upload(st.q, dir + "/q.bin", (size_t)st.B * st.H_q * st.D * e);
        upload(st.k_pool, dir + "/k_pool.bin", st.pool_bytes());
        upload(st.v_pool, dir + "/v_pool.bin", st.pool_bytes());
        upload(st.bt, dir + "/block_tables.bin", (size_t)st.B * st.W * 4);
        if (st.append) {
            upload(st.k_new, dir + "/k_new.bin", (size_t)st.B * st.H_kv * st.D * e);
            upload(st.v_new, dir + "/v_new.bin", (size_t)st.B * st.H_kv * st.D * e);
            upload(st.pos, dir + "/positions.bin", (size_t)st.B * 4);
        } else {
            upload(st.ctx, dir + "/context_lens.bin", (size_t)st.B * 4);
        }
        hipStream_t s = r.count ? masked_stream(n_cus, r.count, r.layout) : nullptr;
        fprintf(stderr, "pkv_cumask: step %s\n", r.tag);
        CHECK_PKV(st.launch(s));
        CHECK_HIP(hipDeviceSynchronize());
        fprintf(stderr, "pkv_cumask: step %s done\n", r.tag);
        std::vector<char> host((size_t)st.B * st.H_q * st.D * 4);
        CHECK_HIP(hipMemcpy(host.data(), st.out, host.size(), hipMemcpyDeviceToHost));
        write_file(dir + "/out_" + r.tag + ".bin", host.data(), host.size());
        host.resize(st.pool_bytes());
        CHECK_HIP(hipMemcpy(host.data(), st.k_pool, host.size(), hipMemcpyDeviceToHost));
        write_file(dir + "/k_pool_" + r.tag + ".bin", host.data(), host.size());
        CHECK_HIP(hipMemcpy(host.data(), st.v_pool, host.size(), hipMemcpyDeviceToHost));
        write_file(dir + "/v_pool_" + r.tag + ".bin", host.data(), host.size());
        if (s) CHECK_PKV(pkv_stream_destroy(s));
    }
    st.release();
    printf("{\"check\": \"ok\", \"n_cus\": %d}\n", n_cus);
    return 0;
}

double elapsed_s(hipEvent_t a, hipEvent_t b) {
    float ms = 0;
    CHECK_HIP(hipEventElapsedTime(&ms, a, b));
    return ms / 1e3;
}

int run_sweep(int argc, char** argv) {
    if (argc < 13) {
        fprintf(stderr, "usage: pkv_cumask sweep dtype B H_q H_kv D P append pool_factor seed steps lens\n");
        return 1;
    }
    const std::string dts = argv[2];
    const int dtype = dts == "f32" ? PKV_F32 : dts == "bf16" ? PKV_BF16 : PKV_F16;
    const int B = atoi(argv[3]), H_q = atoi(argv[4]), H_kv = atoi(argv[5]), D = atoi(argv[6]), P = atoi(argv[7]);
    const bool append = atoi(argv[8]) != 0;
    const double pool_factor = atof(argv[9]);
    const uint64_t seed = strtoull(argv[10], nullptr, 10);
    const int steps = atoi(argv[11]);
    std::vector<int32_t> lens;
    for (const char* p = argv[12]; *p;) {
        lens.push_back((int32_t)strtol(p, (char**)&p, 10));
        if (*p == ',') ++p;
    }
    if ((int)lens.size() != B) {
        fprintf(stderr, "%zu lengths for B = %d\n", lens.size(), B);
        return 1;
    }
    const int e = elem_bytes(dtype);
    int64_t need = 0;
    int W = 1, max_ctx = 0;
    for (int32_t n : lens) {
        need += (n + 15) / 16;
        W = std::max(W, (n + 15) / 16);
        max_ctx = std::max(max_ctx, (int)n);
    }
    const int n_blocks = (int)std::max<int64_t>(need, (int64_t)std::ceil(pool_factor * (double)need));
    double kv_read = 0;
    for (int32_t n : lens) kv_read += (double)(append ? n - 1 : n) * 2.0 * H_kv * D * e;
    const double bytes_per_step = kv_read + (double)B * H_q * D * (e + 4) +
                                  (append ? 4.0 * B * H_kv * D * e : 0.0) + 4.0 * B * (W + 1);
    const int R = std::max(2, (int)std::ceil(4.0 * 256e6 / kv_read));

    // R resident copies of the inputs; block ids scattered by a seeded permutation
    std::vector<Step> sets(R);
    for (int r = 0; r < R; ++r) {
        Step& st = sets[r];
        st.dtype = dtype;
        st.B = B;
        st.H_q = H_q;
        st.H_kv = H_kv;
        st.D = D;
        st.n_blocks = n_blocks;
        st.W = W;
        st.P = P;
        st.max_ctx = max_ctx;
        st.append = append;
        st.scale = 1.0f / std::sqrt((float)D);
        st.alloc();
        fill(st.q, (size_t)B * H_q * D * e, seed * 7 + r, dtype);
        fill(st.k_pool, st.pool_bytes(), seed * 7 + r + 100, dtype);
        fill(st.v_pool, st.pool_bytes(), seed * 7 + r + 200, dtype);
        fill(st.k_new, (size_t)B * H_kv * D * e, seed * 7 + r + 300, dtype);
        fill(st.v_new, (size_t)B * H_kv * D * e, seed * 7 + r + 400, dtype);
        std::vector<int32_t> perm(n_blocks);
        for (int i = 0; i < n_blocks; ++i) perm[i] = i;
        for (int i = n_blocks - 1; i > 0; --i) std::swap(perm[i], perm[mix64(seed + r * 1000003ull + i) % (uint64_t)(i + 1)]);
        std::vector<int32_t> bt((size_t)B * W, -1), pos(B), ctx(B);
        int64_t off = 0;
        for (int b = 0; b < B; ++b) {
            const int nb = (lens[b] + 15) / 16;
            for (int j = 0; j < nb; ++j) bt[(size_t)b * W + j] = perm[off++];
            pos[b] = lens[b] - 1;
            ctx[b] = lens[b];
        }
        CHECK_HIP(hipMemcpy(st.bt, bt.data(), bt.size() * 4, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(st.pos, pos.data(), (size_t)B * 4, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(st.ctx, ctx.data(), (size_t)B * 4, hipMemcpyHostToDevice));
    }
    CHECK_HIP(hipDeviceSynchronize());
    const int n_cus = pkv_device_cu_count();
    const int K = std::max(steps, 2 * R);
    hipEvent_t e0, e1, g0, g1;
    CHECK_HIP(hipEventCreate(&e0));
    CHECK_HIP(hipEventCreate(&e1));
    CHECK_HIP(hipEventCreate(&g0));
    CHECK_HIP(hipEventCreate(&g1));

    auto launch_steps = [&](hipStream_t s, int n) {
        for (int k = 0; k < n; ++k) CHECK_PKV(sets[k % R].launch(s));
    };
    auto time_steps = [&](hipStream_t s) {
        launch_steps(s, R);
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipEventRecord(e0, s));
        launch_steps(s, K);
        CHECK_HIP(hipEventRecord(e1, s));
        CHECK_HIP(hipDeviceSynchronize());
        return elapsed_s(e0, e1) / K;
    };

    std::string sweep = "[";
    double full_bw = 0;
    const int counts[] = {8, 16, 32, 48, 64, 96, 128, 192, 256};
    std::vector<std::string> rows;
    std::vector<double> bws;
    for (int layout = 1; layout >= 0; --layout) {
        for (int c : counts) {
            if (c > n_cus) continue;
            hipStream_t s = masked_stream(n_cus, c, layout);
            const double t = time_steps(s);
            CHECK_PKV(pkv_stream_destroy(s));
            const double bw = bytes_per_step / t / 1e9;
            if (c == n_cus) full_bw = std::max(full_bw, bw);
            char buf[256];
            snprintf(buf, sizeof buf, "{\"cus\": %d, \"layout\": \"%s\", \"us_per_step\": %.2f, \"GBps\": %.1f",
                     c, layout ? "spread" : "first", t * 1e6, bw);
            rows.push_back(buf);
            bws.push_back(bw);
            fprintf(stderr, "sweep %s\n", buf);
        }
    }
    for (size_t i = 0; i < rows.size(); ++i) {
        char buf[64];
        snprintf(buf, sizeof buf, ", \"frac_of_all_cus\": %.3f}", bws[i] / full_bw);
        sweep += (i ? ", " : "") + rows[i] + buf;
    }
    sweep += "]";

    // GEMM beside the attention step
    const int M = 8192;
    void *A = nullptr, *Bm = nullptr, *C = nullptr;
    CHECK_HIP(hipMalloc(&A, (size_t)M * M * 2));
    CHECK_HIP(hipMalloc(&Bm, (size_t)M * M * 2));
    CHECK_HIP(hipMalloc(&C, (size_t)M * M * 2));
    fill(A, (size_t)M * M * 2, seed + 900, PKV_BF16);
    fill(Bm, (size_t)M * M * 2, seed + 901, PKV_BF16);
    CHECK_HIP(hipDeviceSynchronize());
    rocblas_handle h;
    if (rocblas_create_handle(&h) != rocblas_status_success) return 5;
    const float alpha = 1.0f, beta = 0.0f;
    const double gemm_flop = 2.0 * M * (double)M * M;
    auto gemm_on = [&](hipStream_t s, int n) {
        rocblas_set_stream(h, s);
        for (int i = 0; i < n; ++i) {
            const rocblas_status r = rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, M, M, M, &alpha, A,
                                                     rocblas_datatype_bf16_r, M, Bm, rocblas_datatype_bf16_r, M, &beta, C,
                                                     rocblas_datatype_bf16_r, M, C, rocblas_datatype_bf16_r, M,
                                                     rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
            if (r != rocblas_status_success) {
                fprintf(stderr, "rocblas_gemm_ex: %d\n", (int)r);
                exit(5);
            }
        }
    };
    auto time_gemm = [&](hipStream_t s) {
        gemm_on(s, 3);
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipEventRecord(g0, s));
        gemm_on(s, 10);
        CHECK_HIP(hipEventRecord(g1, s));
        CHECK_HIP(hipDeviceSynchronize());
        return elapsed_s(g0, g1) / 10;
    };
    auto corun = [&](hipStream_t sa, hipStream_t sg, const char* a_cus, const char* g_cus) {
        const double ta = time_steps(sa), tg = time_gemm(sg);
        const int n_gemm = std::max(4, (int)std::ceil(K * ta / tg * 1.5) + 2);
        launch_steps(sa, R);
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipEventRecord(g0, sg));
        gemm_on(sg, 2);
        CHECK_HIP(hipEventRecord(e0, sa));
        launch_steps(sa, K);
        CHECK_HIP(hipEventRecord(e1, sa));
        gemm_on(sg, n_gemm - 2);
        CHECK_HIP(hipEventRecord(g1, sg));
        CHECK_HIP(hipDeviceSynchronize());
        const double ta2 = elapsed_s(e0, e1) / K, tg2 = elapsed_s(g0, g1) / n_gemm;
        char buf[512];
        snprintf(buf, sizeof buf,
                 "{\"attention_cus\": %s, \"gemm_cus\": %s, \"attention_alone_GBps\": %.1f, \"gemm_alone_TFLOPs\": %.1f, "
                 "\"attention_corun_GBps\": %.1f, \"gemm_corun_TFLOPs\": %.1f}",
                 a_cus, g_cus, bytes_per_step / ta / 1e9, gemm_flop / tg / 1e12, bytes_per_step / ta2 / 1e9,
                 gemm_flop / tg2 / 1e12);
        fprintf(stderr, "corun %s\n", buf);
        return std::string(buf);
    };
    std::string co = "[";
    const int words = (n_cus + 31) / 32;
    for (int c : {32, 64, 96, 128}) {
        if (c >= n_cus) continue;
        std::vector<uint32_t> ma(words), all(words), mg(words);
        CHECK_PKV(pkv_cu_mask(n_cus, c, 1, ma.data(), words));
        CHECK_PKV(pkv_cu_mask(n_cus, n_cus, 0, all.data(), words));
        for (int w = 0; w < words; ++w) mg[w] = all[w] & ~ma[w];
        void *sa = nullptr, *sg = nullptr;
        CHECK_PKV(pkv_stream_create_cu_masked(ma.data(), words, &sa));
        CHECK_PKV(pkv_stream_create_cu_masked(mg.data(), words, &sg));
        const std::string a = std::to_string(c), g = std::to_string(n_cus - c);
        co += (co.size() > 1 ? ", " : "") + corun((hipStream_t)sa, (hipStream_t)sg, a.c_str(), g.c_str());
        CHECK_PKV(pkv_stream_destroy(sa));
        CHECK_PKV(pkv_stream_destroy(sg));
    }
    {
        hipStream_t sa, sg;
        CHECK_HIP(hipStreamCreateWithFlags(&sa, hipStreamNonBlocking));
        CHECK_HIP(hipStreamCreateWithFlags(&sg, hipStreamNonBlocking));
        co += ", " + corun(sa, sg, "\"all (shared)\"", "\"all (shared)\"");
        CHECK_HIP(hipStreamDestroy(sa));
        CHECK_HIP(hipStreamDestroy(sg));
    }
    co += "]";
    rocblas_destroy_handle(h);
    CHECK_HIP(hipFree(A));
    CHECK_HIP(hipFree(Bm));
    CHECK_HIP(hipFree(C));
    for (Step& st : sets) st.release();
    printf("{\"n_cus\": %d, \"steps_per_point\": %d, \"rotation_sets\": %d, \"bytes_per_step\": %.0f, "
           "\"sweep\": %s, \"corun_gemm_bf16_8192\": %s}\n",
           n_cus, K, R, bytes_per_step, sweep.c_str(), co.c_str());
    return 0;
}

}  // namespace

int main(int argc, char** argv) {
    // unbuffered: a run that dies part-way leaves every line it got to in the parent's pipes
    setvbuf(stdout, nullptr, _IONBF, 0);
    setvbuf(stderr, nullptr, _IONBF, 0);
    fprintf(stderr, "pkv_cumask: start\n");
    if (argc >= 3 && std::string(argv[1]) == "check") return run_check(argv[2]);
    if (argc >= 2 && std::string(argv[1]) == "sweep") return run_sweep(argc, argv);
    fprintf(stderr, "usage: pkv_cumask check DIR | pkv_cumask sweep dtype B H_q H_kv D P append pool_factor seed steps lens\n");
    return 1;
}
