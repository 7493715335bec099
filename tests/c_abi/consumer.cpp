// A consumer of libgdn's C ABI with no Python and no torch: it reads raw
// arrays from a directory, copies them to device memory it allocates itself,
// runs one entry point on a stream of its own and writes the results back as
// raw arrays. The GPU test that drives it compares its outputs with the fp64
// oracle and with the Python binding's.
//
//   consumer MODE DIR B T H Hk K V N_SEQS SCALE L2NORM HAS_S0
//
// MODE chunk_fwd reads q.bin, k.bin (bf16 [B*T, Hk, K]), v.bin (bf16
// [B*T, H, V]), g.bin, beta.bin (fp32 [B*T, H]); MODE prefill reads x.bin
// (bf16 [B*T, C], C = 2 Hk K + H V), w.bin (bf16 [C, 4]), a.bin, b.bin
// (bf16 [B*T, H]), A_log.bin, dt_bias.bin (fp32 [H]). Both read S0.bin (fp32
// [N, H, K, V]) when HAS_S0 is 1 and cu.bin (int32 [N_SEQS + 1]) when N_SEQS
// is above 0, and write o.bin (bf16 [B*T, H, V]) and sf.bin (fp32
// [N, H, K, V]). Exit status: 0 on success, 2 on a HIP error, 3 on a library
// status other than GDN_OK, 1 on bad arguments or files.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gdn.h"

#define HIP_OK(x)                                                                      \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
            std::exit(2);                                                              \
        }                                                                              \
    } while (0)

static std::vector<char> read_all(const std::string& path, size_t expect) {
    std::FILE* f = std::fopen(path.c_str(), "rb");
    if (!f) { std::fprintf(stderr, "cannot open %s\n", path.c_str()); std::exit(1); }
    std::vector<char> buf(expect);
    const size_t got = expect ? std::fread(buf.data(), 1, expect, f) : 0;
    const bool more = std::fgetc(f) != EOF;
    std::fclose(f);
    if (got != expect || more) {
        std::fprintf(stderr, "%s: expected %zu bytes\n", path.c_str(), expect);
        std::exit(1);
    }
    return buf;
}

static void write_all(const std::string& path, const void* p, size_t n) {
    std::FILE* f = std::fopen(path.c_str(), "wb");
    if (!f || (n && std::fwrite(p, 1, n, f) != n)) {
        std::fprintf(stderr, "cannot write %s\n", path.c_str());
        std::exit(1);
    }
    std::fclose(f);
}

// device copy of a host file of `bytes` bytes (at least one byte is allocated)
static void* upload(const std::string& path, size_t bytes) {
    const std::vector<char> h = read_all(path, bytes);
    void* d = nullptr;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
    if (bytes) HIP_OK(hipMemcpy(d, h.data(), bytes, hipMemcpyHostToDevice));
    return d;
}

int main(int argc, char** argv) {
    if (argc != 13) {
        std::fprintf(stderr, "usage: %s chunk_fwd|prefill DIR B T H Hk K V N_SEQS SCALE L2NORM HAS_S0\n",
                     argv[0]);
        return 1;
    }
    const std::string mode = argv[1], dir = std::string(argv[2]) + "/";
    const int B = std::atoi(argv[3]), T = std::atoi(argv[4]), H = std::atoi(argv[5]);
    const int Hk = std::atoi(argv[6]), K = std::atoi(argv[7]), V = std::atoi(argv[8]);
    const int n_seqs = std::atoi(argv[9]);
    const float scale = (float)std::atof(argv[10]);
    const int l2norm = std::atoi(argv[11]), has_s0 = std::atoi(argv[12]);
    if (mode != "chunk_fwd" && mode != "prefill") { std::fprintf(stderr, "unknown mode\n"); return 1; }
    const int64_t rows = (int64_t)B * T;
    const int N = n_seqs > 0 ? n_seqs : B;
    const size_t state_bytes = (size_t)N * H * K * V * sizeof(float);
    const size_t o_bytes = (size_t)rows * H * V * 2;

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    void* S0 = has_s0 ? upload(dir + "S0.bin", state_bytes) : nullptr;
    void* cu = n_seqs > 0 ? upload(dir + "cu.bin", (size_t)(n_seqs + 1) * 4) : nullptr;
    void* Sf = nullptr;
    void* o = nullptr;
    HIP_OK(hipMalloc(&Sf, state_bytes ? state_bytes : 1));
    HIP_OK(hipMalloc(&o, o_bytes ? o_bytes : 1));

    int rc;
    std::vector<void*> inputs;
    if (mode == "chunk_fwd") {
        void* q = upload(dir + "q.bin", (size_t)rows * Hk * K * 2);
        void* k = upload(dir + "k.bin", (size_t)rows * Hk * K * 2);
        void* v = upload(dir + "v.bin", (size_t)rows * H * V * 2);
        void* g = upload(dir + "g.bin", (size_t)rows * H * 4);
        void* beta = upload(dir + "beta.bin", (size_t)rows * H * 4);
        inputs = {q, k, v, g, beta};
        const size_t ws_bytes = gdn_chunk_fwd_workspace_size(B, T, H, Hk, K, V, n_seqs, GDN_BF16);
        void* ws = nullptr;
        HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 1));
        inputs.push_back(ws);
        rc = gdn_chunk_fwd(q, k, (int64_t)Hk * K, v, (int64_t)H * V, (const float*)g, (const float*)beta,
                           (const float*)S0, (float*)Sf, o, (const int32_t*)cu, n_seqs, B, T, H, Hk, K, V,
                           scale, l2norm, GDN_BF16, ws, ws_bytes, (void*)stream);
    } else {
        const int64_t C = 2 * (int64_t)Hk * K + (int64_t)H * V;
        void* x = upload(dir + "x.bin", (size_t)rows * C * 2);
        void* w = upload(dir + "w.bin", (size_t)C * 4 * 2);
        void* a = upload(dir + "a.bin", (size_t)rows * H * 2);
        void* b = upload(dir + "b.bin", (size_t)rows * H * 2);
        void* A_log = upload(dir + "A_log.bin", (size_t)H * 4);
        void* dt_bias = upload(dir + "dt_bias.bin", (size_t)H * 4);
        inputs = {x, w, a, b, A_log, dt_bias};
        const size_t ws_bytes = gdn_prefill_workspace_size(B, T, H, Hk, K, V, n_seqs, GDN_BF16);
        void* ws = nullptr;
        HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 1));
        inputs.push_back(ws);
        rc = gdn_prefill(x, C, w, nullptr, a, H, b, H, (const float*)A_log, (const float*)dt_bias,
                         (const float*)S0, (float*)Sf, o, (const int32_t*)cu, n_seqs, B, T, H, Hk, K, V,
                         scale, l2norm, GDN_BF16, ws, ws_bytes, (void*)stream);
    }
    if (rc != GDN_OK) {
        std::fprintf(stderr, "%s: %s\n", mode.c_str(), gdn_status_string(rc));
        return 3;
    }
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<char> ho(o_bytes), hs(state_bytes);
    if (o_bytes) HIP_OK(hipMemcpy(ho.data(), o, o_bytes, hipMemcpyDeviceToHost));
    if (state_bytes) HIP_OK(hipMemcpy(hs.data(), Sf, state_bytes, hipMemcpyDeviceToHost));
    write_all(dir + "o.bin", ho.data(), o_bytes);
    write_all(dir + "sf.bin", hs.data(), state_bytes);

    for (void* p : inputs) HIP_OK(hipFree(p));
    if (S0) HIP_OK(hipFree(S0));
    if (cu) HIP_OK(hipFree(cu));
    HIP_OK(hipFree(Sf));
    HIP_OK(hipFree(o));
    HIP_OK(hipStreamDestroy(stream));
    std::printf("%s ok\n", mode.c_str());
    return 0;
}
