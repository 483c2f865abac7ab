// Host-only driver for the C ABI's argument validation (gdn_api.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_asan_host.py.  The
// launchers are stubs that record what they were handed, so every entry point runs
// its checks, its pointer arithmetic and its routing without a GPU; each case checks
// the status, the message and (for valid calls) what reached the launchers.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "stub HIP error"; }

namespace gdn {
static int n_decode = 0, n_prefill = 0;
static DecodeArgs last_decode;
static PrefillArgs last_prefill;
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
    ++n_decode;
    last_decode = a;
    return hipSuccess;
}
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t) {
    ++n_prefill;
    last_prefill = a;
    return hipSuccess;
}
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) { return launch_prefill(a, s); }
size_t prefill_workspace_bytes(int, int, int, int64_t) { return 0; }
}  // namespace gdn

static int failures = 0;
#define CHECK(cond, ...)                                            \
    do {                                                            \
        if (!(cond)) {                                              \
            ++failures;                                             \
            std::fprintf(stderr, "FAIL line %d: ", __LINE__);       \
            std::fprintf(stderr, __VA_ARGS__);                      \
            std::fprintf(stderr, "\n");                             \
        }                                                           \
    } while (0)

static void expect(gdn_status got, gdn_status want, const char* needle, int line) {
    if (got != want) {
        ++failures;
        std::fprintf(stderr, "FAIL line %d: status %d, expected %d (%s)\n", line, got, want, gdn_last_error());
        return;
    }
    const char* msg = gdn_last_error();
    if (want == GDN_OK && msg[0] != '\0') {
        ++failures;
        std::fprintf(stderr, "FAIL line %d: OK with a message '%s'\n", line, msg);
    }
    if (want != GDN_OK && (msg[0] == '\0' || (needle && !std::strstr(msg, needle)))) {
        ++failures;
        std::fprintf(stderr, "FAIL line %d: message '%s' lacks '%s'\n", line, msg, needle ? needle : "");
    }
}
#define EXPECT(call, want, needle) expect((call), (want), (needle), __LINE__)

int main() {
    // host buffers stand in for device memory: nothing is dereferenced by the library
    std::vector<uint8_t> arena(1 << 20);
    auto at = [&](size_t off) { return static_cast<void*>(arena.data() + 256 + off); };
    void* q = at(0);
    void* k = at(4096);
    void* v = at(8192);
    float* g = static_cast<float*>(at(16384));
    float* beta = static_cast<float*>(at(20480));
    void* o = at(24576);
    float* pool = static_cast<float*>(at(32768));
    int32_t* si = static_cast<int32_t*>(at(65536));
    int32_t* so = static_cast<int32_t*>(at(65536 + 1024));
    int32_t* cu = static_cast<int32_t*>(at(65536 + 2048));
    int32_t* init = static_cast<int32_t*>(at(65536 + 3072));
    int32_t* fin = static_cast<int32_t*>(at(65536 + 4096));
    int32_t* offs = static_cast<int32_t*>(at(65536 + 5120));
    float* exps = static_cast<float*>(at(131072));
    void* odd = at(4096 + 2);   // misaligned

    gdn_shape sh = {2, 4, 128, 128, GDN_BF16, 0.088f};
    hipStream_t st = nullptr;

    // ---- shapes
    gdn_shape bad = sh;
    bad.num_k_heads = 0;
    EXPECT(gdn_recurrent_decode(&bad, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "head counts");
    bad = sh; bad.num_v_heads = 6; bad.num_k_heads = 4;
    EXPECT(gdn_recurrent_decode(&bad, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_UNSUPPORTED, "not a multiple");
    bad = sh; bad.d_k = 96;
    EXPECT(gdn_recurrent_decode(&bad, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_UNSUPPORTED, "head dims");
    bad = sh; bad.dtype = 7;
    EXPECT(gdn_recurrent_decode(&bad, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_UNSUPPORTED, "dtype");
    bad = sh; bad.scale = 1.0f / 0.0f;
    EXPECT(gdn_recurrent_decode(&bad, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "scale");
    EXPECT(gdn_recurrent_decode(nullptr, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "shape");
    CHECK(gdn::n_decode == 0, "a rejected call launched");

    // ---- decode
    EXPECT(gdn_recurrent_decode(&sh, -1, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "num_rows");
    EXPECT(gdn_recurrent_decode(&sh, 4, nullptr, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "q is NULL");
    EXPECT(gdn_recurrent_decode(&sh, 4, odd, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "aligned");
    EXPECT(gdn_recurrent_decode(&sh, 4, q, k, v, g, beta, o, pool, 8, si, nullptr, st), GDN_ERR_INVALID_ARGUMENT, "slot_out");
    EXPECT(gdn_recurrent_decode(&sh, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr,
                                nullptr, st), GDN_OK, nullptr);
    CHECK(gdn::n_decode == 0, "zero rows launched");
    EXPECT(gdn_recurrent_decode(&sh, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_OK, nullptr);
    CHECK(gdn::n_decode == 1 && gdn::last_decode.num_rows == 4 && gdn::last_decode.tokens_per_row == 1 &&
              gdn::last_decode.q == q && gdn::last_decode.slot_out == so && gdn::last_decode.H_v == 4,
          "decode arguments did not reach the launcher");

    // ---- verify
    EXPECT(gdn_recurrent_verify(&sh, 4, 0, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_INVALID_ARGUMENT, "tokens_per_row");
    EXPECT(gdn_recurrent_verify(&sh, 1 << 30, 4, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_ERR_UNSUPPORTED, "too large");
    EXPECT(gdn_recurrent_verify(&sh, 4, 3, q, k, v, g, beta, o, pool, 8, si, so, st), GDN_OK, nullptr);
    CHECK(gdn::n_decode == 2 && gdn::last_decode.tokens_per_row == 3, "verify did not route to the decode launcher");

    // ---- prefill
    auto prefill = [&](const gdn_shape* s, int N, int64_t T, int grid, size_t ws_bytes, void* ws, const int32_t* cu_,
                       const void* q_, float* exp_) {
        return gdn_chunk_prefill(s, N, T, cu_, q_, k, v, g, beta, o, pool, 8, init, fin, nullptr, grid, exp_, offs,
                                 nullptr, 4, ws, ws_bytes, st);
    };
    EXPECT(prefill(&sh, -1, 10, 0, 0, nullptr, cu, q, nullptr), GDN_ERR_INVALID_ARGUMENT, "num_seqs");
    EXPECT(prefill(&sh, 2, -5, 0, 0, nullptr, cu, q, nullptr), GDN_ERR_INVALID_ARGUMENT, "total_tokens");
    EXPECT(prefill(&sh, 2, (int64_t)1 << 40, 0, 0, nullptr, cu, q, nullptr), GDN_ERR_UNSUPPORTED, "total_tokens");
    EXPECT(prefill(&sh, 2, 100, 1056, 0, nullptr, cu, q, exps), GDN_ERR_INVALID_ARGUMENT, "multiple of chunk size 64");
    EXPECT(prefill(&sh, 2, 100, -64, 0, nullptr, cu, q, exps), GDN_ERR_INVALID_ARGUMENT, "export_grid");
    EXPECT(prefill(&sh, 2, 100, 0, 0, nullptr, nullptr, q, nullptr), GDN_ERR_INVALID_ARGUMENT, "cu_seqlens");
    EXPECT(prefill(&sh, 2, 100, 0, 0, nullptr, cu, nullptr, nullptr), GDN_ERR_INVALID_ARGUMENT, "q is NULL");
    EXPECT(prefill(&sh, 2, 100, 64, 0, nullptr, cu, q, nullptr), GDN_ERR_INVALID_ARGUMENT, "export_states");
    CHECK(gdn::n_prefill == 0, "a rejected prefill launched");
    EXPECT(prefill(&sh, 0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr), GDN_OK, nullptr);
    CHECK(gdn::n_prefill == 0, "an empty prefill launched");
    EXPECT(prefill(&sh, 2, 100, 1088, 0, nullptr, cu, q, exps), GDN_OK, nullptr);
    CHECK(gdn::n_prefill == 1 && gdn::last_prefill.num_seqs == 2 && gdn::last_prefill.total_tokens == 100 &&
              gdn::last_prefill.export_grid == 1088 && gdn::last_prefill.export_states == exps &&
              gdn::last_prefill.export_capacity == 4,
          "prefill arguments did not reach the launcher");
    CHECK(gdn_chunk_prefill_workspace_size(&sh, 2, 100) == 0, "workspace size");
    CHECK(gdn_chunk_prefill_workspace_size(nullptr, 2, 100) == 0, "workspace size of a NULL shape");

    // ---- mixed step: the prefill part starts num_decode_rows tokens in
    EXPECT(gdn_mixed_step(&sh, 3, si, so, 2, 100, cu, q, k, v, g, beta, o, pool, 8, init, fin, nullptr, 0, nullptr,
                          nullptr, nullptr, 0, nullptr, 0, st), GDN_OK, nullptr);
    const size_t esz = 2;
    CHECK(gdn::n_decode == 3 && gdn::last_decode.num_rows == 3, "mixed step decode part");
    CHECK(gdn::n_prefill == 2 &&
              gdn::last_prefill.q == static_cast<const char*>(q) + 3 * sh.num_k_heads * sh.d_k * esz &&
              gdn::last_prefill.v == static_cast<const char*>(v) + 3 * sh.num_v_heads * sh.d_v * esz &&
              gdn::last_prefill.g == g + 3 * sh.num_v_heads && gdn::last_prefill.o ==
              static_cast<char*>(o) + 3 * sh.num_v_heads * sh.d_v * esz,
          "mixed step prefill pointers are not offset by the decode rows");
    EXPECT(gdn_mixed_step(&sh, 3, si, nullptr, 2, 100, cu, q, k, v, g, beta, o, pool, 8, init, fin, nullptr, 0,
                          nullptr, nullptr, nullptr, 0, nullptr, 0, st), GDN_ERR_INVALID_ARGUMENT, "slot_out");
    CHECK(gdn::n_decode == 3 && gdn::n_prefill == 2, "a rejected mixed step launched");
    EXPECT(gdn_mixed_step(&sh, 0, nullptr, nullptr, 0, 0, nullptr, q, k, v, g, beta, o, pool, 8, nullptr, nullptr,
                          nullptr, 0, nullptr, nullptr, nullptr, 0, nullptr, 0, st), GDN_OK, nullptr);
    CHECK(gdn::n_decode == 3 && gdn::n_prefill == 2, "an empty mixed step launched");

    if (failures) {
        std::fprintf(stderr, "%d validation checks failed\n", failures);
        return 1;
    }
    std::printf("validation driver: all checks passed\n");
    return 0;
}
