// Host-to-device copies of pageable host memory through two pinned buffers
// that this object allocates (hipHostMalloc) and frees.  The host copies a
// chunk into one buffer while the DMA engine drains the other, so the
// runtime's own pageable-copy path (its staging pool, shared by every thread
// of the process) is never used for the large uploads of grammar images and
// CSR arrays, which several worker threads issue at once.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstring>

namespace gcs {

class PinnedStage {
  public:
    static constexpr size_t kChunk = size_t(16) << 20;

    PinnedStage() = default;
    PinnedStage(const PinnedStage&) = delete;
    PinnedStage& operator=(const PinnedStage&) = delete;
    ~PinnedStage()
    {
        for (int i = 0; i < 2; ++i) {
            if (used_[i]) (void)hipEventSynchronize(ev_[i]);
            if (ev_[i]) (void)hipEventDestroy(ev_[i]);
            if (buf_[i]) (void)hipHostFree(buf_[i]);
        }
    }

    hipError_t init()
    {
        for (int i = 0; i < 2; ++i) {
            hipError_t e = hipHostMalloc((void**)&buf_[i], kChunk, hipHostMallocDefault);
            if (e != hipSuccess) {
                buf_[i] = nullptr;
                return e;
            }
            e = hipEventCreateWithFlags(&ev_[i], hipEventDisableTiming);
            if (e != hipSuccess) {
                ev_[i] = nullptr;
                return e;
            }
        }
        return hipSuccess;
    }

    // Queue dst (device) <- src (host, bytes) on stream s.  The source may be
    // reused when this returns; the destination is complete once the stream
    // has reached this point.
    hipError_t h2d(void* dst, const void* src, size_t bytes, hipStream_t s)
    {
        auto* d = (unsigned char*)dst;
        auto* h = (const unsigned char*)src;
        for (size_t off = 0; off < bytes; off += kChunk) {
            const size_t n = std::min(kChunk, bytes - off);
            const int i = next_;
            if (used_[i]) {
                const hipError_t e = hipEventSynchronize(ev_[i]);  // its previous chunk has left
                if (e != hipSuccess) return e;
            }
            std::memcpy(buf_[i], h + off, n);
            hipError_t e = hipMemcpyAsync(d + off, buf_[i], n, hipMemcpyHostToDevice, s);
            if (e == hipSuccess) e = hipEventRecord(ev_[i], s);
            if (e != hipSuccess) return e;
            used_[i] = true;
            next_ ^= 1;
        }
        return hipSuccess;
    }

  private:
    unsigned char* buf_[2] = {nullptr, nullptr};
    hipEvent_t ev_[2] = {nullptr, nullptr};
    bool used_[2] = {false, false};
    int next_ = 0;
};

}  // namespace gcs
