// ds_workspace.hpp -- the cache of library-owned split workspaces.
//
// Host code only, independent of HIP: the stream synchronisation, free and
// allocation calls come from the Ops type (the library's uses HIP; the CPU
// tests use fake streams that check every free against the uses still
// queued).
//
// One workspace per (device, stream), and per thread as well for a stream
// handle that names a different stream in every thread (hipStreamPerThread).
// A caller holds mu() from acquire() until its kernels are queued, so a
// concurrent call that grows (frees) the same workspace waits for them to be
// queued, and then synchronises the stream before the free: no queued kernel
// ever uses freed memory.
#pragma once

#include <stddef.h>

#include <map>
#include <mutex>
#include <thread>
#include <tuple>

namespace ds {

struct WsBuf {
    void* ptr = nullptr;
    size_t bytes = 0;
    bool zeroed = false;  // its reserved shared-threshold cells have been cleared
};

// Ops provides:
//   bool per_thread(void* stream)         the handle names a stream per thread
//   int  sync(void* stream)               wait for the stream's queued work (0: ok)
//   int  release(void* ptr)               free device memory (0: ok)
//   int  allocate(void** ptr, size_t n)   allocate device memory (0: ok)
template <class Ops>
class WsCache {
  public:
    std::mutex& mu() { return mu_; }

    // The workspace of (dev, stream) with at least `bytes`, grown if needed:
    // the stream is synchronised before the old buffer is freed. The caller
    // holds mu(). Returns 0, or the failing Ops call's status (the entry is
    // then empty).
    int acquire(Ops& ops, int dev, void* stream, size_t bytes, WsBuf** out) {
        const std::thread::id tid = ops.per_thread(stream) ? std::this_thread::get_id() : std::thread::id();
        WsBuf& w = bufs_[std::make_tuple(dev, stream, tid)];
        if (w.bytes < bytes) {
            if (w.ptr) {
                if (int st = ops.sync(stream)) return st;
                if (int st = ops.release(w.ptr)) return st;
                w.ptr = nullptr;
                w.bytes = 0;
            }
            w.zeroed = false;
            void* ptr = nullptr;
            if (int st = ops.allocate(&ptr, bytes)) return st;
            w.ptr = ptr;
            w.bytes = bytes;
        }
        *out = &w;
        return 0;
    }

    // Free every workspace (no call using one may still be queued). Takes mu().
    void release_all(Ops& ops) {
        std::lock_guard<std::mutex> lk(mu_);
        for (auto& kv : bufs_) {
            if (kv.second.ptr) (void)ops.release(kv.second.ptr);
        }
        bufs_.clear();
    }

  private:
    std::mutex mu_;
    std::map<std::tuple<int, void*, std::thread::id>, WsBuf> bufs_;
};

}  // namespace ds
