// The workspace cache (csrc/ds_workspace.hpp) under many threads, with fake
// streams. Every call takes the cache's lock, acquires a workspace and queues
// a use of it on its stream before unlocking, as the library queues its
// kernels; a stream completes its queued uses only when synchronised. The
// check fails on a free of a buffer that a queued use still holds, on a use of
// a buffer smaller than it asked for, on a use of a freed buffer, and (under
// AddressSanitizer) on a leak. Two handles are shared by all threads, and one
// names a different stream in every thread, as hipStreamPerThread does.
#include "../top_selection_row_amd/csrc/ds_workspace.hpp"

#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <map>
#include <memory>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

namespace {

std::atomic<int> g_errors{0};
#define CHECK(c)                                                               \
    do {                                                                       \
        if (!(c)) {                                                            \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);    \
            ++g_errors;                                                        \
        }                                                                      \
    } while (0)

struct Use {
    void* ptr;
    size_t bytes;
};
struct FakeStream {
    std::mutex mu;
    std::vector<Use> queued;
};

constexpr int kThreads = 8;
constexpr int kCalls = 3000;

struct FakeOps {
    std::mutex mu;                  // guards live
    std::map<void*, size_t> live;   // allocated buffers and their sizes
    FakeStream shared[2];           // handles every thread uses
    std::unique_ptr<FakeStream> own[kThreads];  // the per-thread handle's streams
    int per_thread_tag = 0;         // its address is the per-thread handle
    static thread_local int me;     // this thread's index

    void* shared_handle(int i) { return &shared[i]; }
    void* per_thread_handle() { return &per_thread_tag; }
    FakeStream* resolve(void* s) {
        return s == per_thread_handle() ? own[me].get() : static_cast<FakeStream*>(s);
    }
    bool per_thread(void* s) const { return s == &per_thread_tag; }

    int sync(void* s) {
        FakeStream* fs = resolve(s);
        std::lock_guard<std::mutex> lk(fs->mu);
        std::lock_guard<std::mutex> lk2(mu);
        for (const Use& u : fs->queued) {
            auto it = live.find(u.ptr);
            CHECK(it != live.end());
            CHECK(it == live.end() || it->second >= u.bytes);
        }
        fs->queued.clear();
        return 0;
    }
    bool queued_anywhere(void* p) {
        std::vector<FakeStream*> all = {&shared[0], &shared[1]};
        for (auto& o : own) all.push_back(o.get());
        for (FakeStream* fs : all) {
            std::lock_guard<std::mutex> lk(fs->mu);
            for (const Use& u : fs->queued)
                if (u.ptr == p) return true;
        }
        return false;
    }
    int release(void* p) {
        CHECK(!queued_anywhere(p));  // freed while a queued use still holds it
        std::lock_guard<std::mutex> lk(mu);
        CHECK(live.erase(p) == 1);
        free(p);
        return 0;
    }
    int allocate(void** p, size_t n) {
        *p = malloc(n);
        std::lock_guard<std::mutex> lk(mu);
        live[*p] = n;
        return 0;
    }
};
thread_local int FakeOps::me = 0;

}  // namespace

int main() {
    FakeOps ops;
    for (auto& o : ops.own) o.reset(new FakeStream);
    ds::WsCache<FakeOps> cache;
    std::vector<std::thread> threads;
    for (int t = 0; t < kThreads; ++t) {
        threads.emplace_back([&, t] {
            FakeOps::me = t;
            std::mt19937 rng(1234u + (unsigned)t);
            for (int c = 0; c < kCalls; ++c) {
                const int pick = (int)(rng() % 3u);
                void* handle = pick == 2 ? ops.per_thread_handle() : ops.shared_handle(pick);
                // sizes that rise through the run, so workspaces keep
                // growing (and freeing) while other threads have uses queued
                const size_t bytes = 256u * (size_t)(1 + c + (int)(rng() % 64u));
                const int dev = (int)(rng() % 2u);
                {
                    std::lock_guard<std::mutex> lk(cache.mu());
                    ds::WsBuf* w = nullptr;
                    CHECK(cache.acquire(ops, dev, handle, bytes, &w) == 0);
                    CHECK(w != nullptr && w->ptr != nullptr && w->bytes >= bytes);
                    FakeStream* fs = ops.resolve(handle);
                    std::lock_guard<std::mutex> lk2(fs->mu);
                    fs->queued.push_back(Use{w->ptr, bytes});  // the call's kernels, queued
                }
                if (rng() % 16u == 0u) ops.sync(handle);  // the stream catches up now and then
            }
            ops.sync(ops.per_thread_handle());
        });
    }
    for (auto& th : threads) th.join();
    ops.sync(ops.shared_handle(0));
    ops.sync(ops.shared_handle(1));
    cache.release_all(ops);
    CHECK(ops.live.empty());
    if (g_errors.load() != 0) {
        fprintf(stderr, "%d checks failed\n", g_errors.load());
        return 1;
    }
    printf("workspace cache: %d threads x %d calls, no free of a queued buffer\n", kThreads, kCalls);
    return 0;
}
