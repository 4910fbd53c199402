// Host-side stress driver for the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
// Eight threads call the host-only entry points at once: validation, the
// stride-phase plan, workspace-size queries, the tile-config table (query,
// save, load, clear) and the per-thread error text. Nothing here launches a
// kernel, so it runs on a machine without a GPU. Exit status 0 means every
// check held and the sanitizers reported nothing.
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "conv2d_dgrad.h"

namespace {

std::atomic<int> g_failures{0};

void expect(bool ok, const char* what, int thread, int iter)
{
    if (!ok) {
        g_failures.fetch_add(1);
        std::fprintf(stderr, "thread %d iteration %d: %s\n", thread, iter, what);
    }
}

// Fake, aligned, non-overlapping device addresses: validation never reads them.
const uintptr_t kDy = 0x10000000, kW = 0x20000000, kDx = 0x30000000, kZ = 0x40000000;

void worker(int t, const std::string& dir)
{
    conv2d_dgrad_phase phases[64];
    const std::string mine = dir + "/table_" + std::to_string(t) + ".txt";
    for (int i = 0; i < 3000; ++i) {
        const int N = 1 + (i + t) % 5, H = 5 + i % 11, W = 4 + (i * 7) % 13;
        const int C = 8 * (1 + i % 9), K = 8 * (1 + (i + 3) % 7);
        const int R = 1 + i % 4, S = 1 + (i / 3) % 4, stride = 1 + i % 5, pad = i % 3;
        switch ((i + t) % 6) {
        case 0: {   // a valid check, then an invalid one: the error text is this thread's own
            int rc = conv2d_dgrad_check((void*)kDy, (void*)kW, (void*)kDx, N, H, W, C, K, R, S, stride, pad, 0,
                                        nullptr);
            const bool valid = (H + 2 * pad - R) >= 0 && (W + 2 * pad - S) >= 0;
            expect(rc == (valid ? CONV2D_DGRAD_OK : CONV2D_DGRAD_INVALID_ARGUMENT), "check code", t, i);
            rc = conv2d_dgrad_check((void*)kDy, (void*)kW, (void*)kDx, N, H, W, C + 4, K, R, S, stride, pad, 0,
                                    nullptr);
            expect(rc != CONV2D_DGRAD_OK && std::strlen(conv2d_dgrad_last_error()) > 0, "error text", t, i);
            rc = conv2d_dgrad_check((void*)kDy, (void*)kW, (void*)(kDy + 16), 2, 8, 8, 16, 8, 3, 3, 1, 1, 0,
                                    nullptr);
            expect(rc == CONV2D_DGRAD_INVALID_ARGUMENT, "overlap detected", t, i);
            rc = conv2d_dgrad_check((void*)kDy, (void*)kW, (void*)kDx, 2, 8, 8, 16, 8, 3, 3, 1, 1, 2, (void*)kZ);
            expect(rc == CONV2D_DGRAD_OK && conv2d_dgrad_last_error()[0] == '\0', "clean error after success", t,
                   i);
            break;
        }
        case 1: {   // the plan: lattices cover dx exactly, heaviest first
            int n = 0, P = 0, Q = 0;
            const int rc = conv2d_dgrad_plan(N, H, W, C, K, R, S, stride, pad, phases, 64, &n, &P, &Q);
            if (rc != CONV2D_DGRAD_OK)
                break;
            long long m = 0;
            int prev = 1 << 30;
            for (int k = 0; k < n && k < 64; ++k) {
                m += phases[k].M;
                const int taps = phases[k].nr * phases[k].nt;
                expect(taps <= prev, "heaviest first", t, i);
                prev = taps;
            }
            expect(m == (long long)N * H * W, "lattices cover dx", t, i);
            break;
        }
        case 2: {   // workspace sizes are 0 or above the counter area
            size_t b = 1;
            int rc = conv2d_dgrad_workspace_size(N, H, W, C, K, R, S, stride, pad, i % 3, &b);
            expect(rc != CONV2D_DGRAD_OK || b == 0 || b > 65536, "dgrad workspace size", t, i);
            rc = conv2d_wgrad_workspace_size(N, H, W, C, K, R, S, stride, pad, &b);
            expect(rc != CONV2D_DGRAD_OK || b == 0 || b > 65536, "wgrad workspace size", t, i);
            break;
        }
        case 3: {   // the table: query
            int id = -1, cached = -1, split = -1;
            const int rc = conv2d_dgrad_query_config(N, H, W, C, K, R, S, stride, pad, 0, i % 2, &id, &cached,
                                                     &split);
            if (rc == CONV2D_DGRAD_OK)
                expect(id >= 0 && id < conv2d_dgrad_num_configs() && (cached == 0 || cached == 1), "query", t, i);
            break;
        }
        case 4: {   // the table: save and load back
            if (conv2d_dgrad_cache_save(mine.c_str()) == CONV2D_DGRAD_OK)
                expect(conv2d_dgrad_cache_load(mine.c_str()) == CONV2D_DGRAD_OK, "load what was saved", t, i);
            expect(conv2d_dgrad_cache_size() >= 0, "size", t, i);
            break;
        }
        default: {  // the table: shared file loads, an occasional clear, the autotune flag
            conv2d_dgrad_cache_load((dir + "/shared.txt").c_str());
            if (i % 40 == 0)
                conv2d_dgrad_cache_clear();
            const int prev_at = conv2d_dgrad_set_autotune(i % 2);
            expect(prev_at == 0 || prev_at == 1, "autotune flag", t, i);
            break;
        }
        }
    }
}

}  // namespace

int main(int argc, char** argv)
{
    if (argc < 2) {
        std::fprintf(stderr, "usage: abi_stress <scratch dir>\n");
        return 2;
    }
    const std::string dir = argv[1];
    {   // a shared table for the loaders: 64 keys on a CPU-only host ("none", 256 CUs)
        char name[64];
        conv2d_dgrad_config_name(0, name, sizeof(name));
        FILE* f = std::fopen((dir + "/shared.txt").c_str(), "w");
        if (!f)
            return 2;
        for (int n = 1; n <= 64; ++n)
            std::fprintf(f, "%d 8 8 16 8 3 3 1 1 0 none 256 %d %s\n", n, n % 2, name);
        std::fputs("a line that is not an entry\n", f);
        std::fclose(f);
    }
    std::vector<std::thread> threads;
    for (int t = 0; t < 8; ++t)
        threads.emplace_back(worker, t, dir);
    for (auto& th : threads)
        th.join();
    conv2d_dgrad_cache_clear();
    expect(conv2d_dgrad_cache_load((dir + "/shared.txt").c_str()) == CONV2D_DGRAD_OK, "final load", -1, 0);
    expect(conv2d_dgrad_cache_size() == 64, "64 entries after the final load", -1, 0);
    conv2d_dgrad_cache_clear();
    std::printf("abi_stress: %d failures\n", g_failures.load());
    return g_failures.load() == 0 ? 0 : 1;
}
