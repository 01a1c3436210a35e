// DMA-engine copies (sdma.cpp), used by the host side (plan.cpp). Not part of
// the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "tide.h"

namespace tide {

// Linear copies on the DMA engines of HIP device `dev` (sdma.cpp): waits for
// the work already enqueued on `stream`, submits the copies spread over every
// engine the device offers for copies inside its memory, and returns once all
// have completed (a bounded wait). No compute unit is used. On a non-OK status
// *err says why.
struct DmaCopy {
    void* dst;
    const void* src;
    uint64_t bytes;
};
struct DmaReport {
    int engines = 0;      // engines used
    int64_t copies = 0;   // copies submitted (after splitting large ones)
    int64_t bytes = 0;    // bytes copied
};
tide_status dma_copies(int dev, hipStream_t stream, const std::vector<DmaCopy>& copies,
                       DmaReport* report, std::string* err);
// Engines dma_copies spreads over on device `dev`.
tide_status dma_engine_count(int dev, int* engines, std::string* err);

}  // namespace tide
