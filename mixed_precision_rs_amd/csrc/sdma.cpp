// Copies on the GPU's DMA (SDMA) engines, through the HSA runtime, for the
// engine of the all-gather placement and of the Slot-Reuse staging that uses
// no compute units (page 1 "The big picture" and "All-gather: parameters land
// at their final address": the all-gather's data movement runs on copy
// engines; page 3 Table 1, all-gather SM budget 0; page 3 Figure 2(b),
// copy-engine staging of bf16 slices).
//
// MI355X offers 14 DMA engines for copies inside one GPU's memory, each
// moving about 60 GB/s; a strided (rect) copy runs on a single engine. So a
// placement is cut into linear copies, one per (parameter, rank) piece, and
// those are spread over every engine (largest first onto the least loaded
// engine); copies larger than a quarter of an even share are split first.
//
// Ordering is done on the host: the work already enqueued on the caller's
// stream is waited for, the copies are submitted with one shared completion
// signal, and the call returns once the signal shows that all of them have
// completed. The wait is bounded; the GPU never waits on a host-side signal.
#include <hsa/hsa.h>
#include <hsa/hsa_ext_amd.h>

#include <algorithm>
#include <chrono>
#include <map>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "sdma.hpp"
#include "tide_internal.hpp"

namespace tide {
namespace {

struct DmaDevice {
    bool ok = false;
    std::string why;                 // reason when !ok
    hsa_agent_t agent{};
    std::vector<uint32_t> engines;   // engine id bits usable for copies inside the device
};

std::mutex g_mu;
bool g_hsa_up = false;
std::map<int, DmaDevice> g_devs;

std::string hsa_text(hsa_status_t s) {
    const char* m = nullptr;
    if (hsa_status_string(s, &m) != HSA_STATUS_SUCCESS || !m) return "HSA status " + std::to_string((int)s);
    return m;
}

hsa_status_t collect_gpus(hsa_agent_t a, void* data) {
    hsa_device_type_t t;
    if (hsa_agent_get_info(a, HSA_AGENT_INFO_DEVICE, &t) == HSA_STATUS_SUCCESS &&
        t == HSA_DEVICE_TYPE_GPU)
        static_cast<std::vector<hsa_agent_t>*>(data)->push_back(a);
    return HSA_STATUS_SUCCESS;
}

// The HSA agent of HIP device `dev` (same PCI domain, bus and device) and its
// DMA engines for device-local copies. Caller holds g_mu.
const DmaDevice& dma_device(int dev) {
    auto it = g_devs.find(dev);
    if (it != g_devs.end()) return it->second;
    DmaDevice d;
    do {
        if (!g_hsa_up) {
            // Reference-counted: the HIP runtime has initialised the same runtime.
            hsa_status_t s = hsa_init();
            if (s != HSA_STATUS_SUCCESS) {
                d.why = "hsa_init: " + hsa_text(s);
                break;
            }
            g_hsa_up = true;
        }
        int bus = -1, devno = -1, dom = -1;
        if (hipDeviceGetAttribute(&bus, hipDeviceAttributePciBusId, dev) != hipSuccess ||
            hipDeviceGetAttribute(&devno, hipDeviceAttributePciDeviceId, dev) != hipSuccess ||
            hipDeviceGetAttribute(&dom, hipDeviceAttributePciDomainID, dev) != hipSuccess) {
            d.why = "the HIP device's PCI location could not be read";
            break;
        }
        std::vector<hsa_agent_t> gpus;
        hsa_status_t s = hsa_iterate_agents(collect_gpus, &gpus);
        if (s != HSA_STATUS_SUCCESS) {
            d.why = "hsa_iterate_agents: " + hsa_text(s);
            break;
        }
        int matches = 0;
        for (hsa_agent_t a : gpus) {
            uint32_t bdf = 0, domain = 0;
            if (hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_BDFID, &bdf) != HSA_STATUS_SUCCESS ||
                hsa_agent_get_info(a, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_DOMAIN, &domain) != HSA_STATUS_SUCCESS)
                continue;
            // BDF id: bus in bits 8-15, device in bits 3-7.
            if ((int)((bdf >> 8) & 0xff) == bus && (int)((bdf >> 3) & 0x1f) == devno && (int)domain == dom) {
                d.agent = a;
                ++matches;
            }
        }
        if (matches != 1) {
            d.why = "HIP device " + std::to_string(dev) + " matches " + std::to_string(matches) +
                    " HSA agents by PCI location (one is needed)";
            break;
        }
        uint32_t mask = 0;
        s = hsa_amd_memory_copy_engine_status(d.agent, d.agent, &mask);
        if (s != HSA_STATUS_SUCCESS || mask == 0) {
            // Runtimes that do not answer for copies inside one agent (the one
            // PyTorch ships answers INVALID_AGENT) still run forced copies on
            // any engine: take the engines meant for device-to-device traffic
            // (the xGMI ones, numbered after the host-link ones), else all.
            uint32_t nh = 0, nx = 0;
            if (hsa_agent_get_info(d.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_ENG, &nh) !=
                    HSA_STATUS_SUCCESS ||
                hsa_agent_get_info(d.agent, (hsa_agent_info_t)HSA_AMD_AGENT_INFO_NUM_SDMA_XGMI_ENG, &nx) !=
                    HSA_STATUS_SUCCESS)
                nh = nx = 0;
            const uint32_t first = nx > 0 ? nh : 0, count = nx > 0 ? nx : nh;
            mask = 0;
            for (uint32_t e = first; e < first + count && e < 16; ++e) mask |= 1u << e;
        }
        if (mask == 0) {
            d.why = "no DMA engine is available for copies inside the device" +
                    (s != HSA_STATUS_SUCCESS ? " (" + hsa_text(s) + ")" : std::string());
            break;
        }
        for (int e = 0; e < 32; ++e)
            if (mask & (1u << e)) d.engines.push_back(1u << e);
        d.ok = true;
    } while (false);
    return g_devs.emplace(dev, d).first->second;
}

// Copies larger than a quarter of an even share of the bytes over the engines
// are split, so that one large piece does not leave the other engines idle; no
// piece is split below this size (one copy costs the host about 0.4 us to
// submit, and 1 MiB takes an engine about 17 us).
constexpr uint64_t kMinSplit = (uint64_t)1 << 20;

}  // namespace

tide_status dma_copies(int dev, hipStream_t stream, const std::vector<DmaCopy>& in,
                       DmaReport* report, std::string* err) {
    const DmaDevice* d;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        d = &dma_device(dev);   // entries are never erased: the pointer stays valid
    }
    if (!d->ok) {
        *err = "the DMA-engine path is not available: " + d->why;
        return TIDE_ERR_UNSUPPORTED;
    }
    const int E = (int)d->engines.size();
    uint64_t total = 0;
    for (const DmaCopy& c : in) total += c.bytes;
    std::vector<DmaCopy> cp;
    cp.reserve(in.size());
    const uint64_t share = (total + (uint64_t)E - 1) / (uint64_t)E;
    const uint64_t cut = std::max<uint64_t>(kMinSplit, (share / 4 + 4095) / 4096 * 4096);
    for (const DmaCopy& c : in) {
        if (c.bytes == 0) continue;
        for (uint64_t off = 0; off < c.bytes; off += cut) {
            const uint64_t n = std::min(cut, c.bytes - off);
            cp.push_back(DmaCopy{static_cast<char*>(c.dst) + off,
                                 static_cast<const char*>(c.src) + off, n});
        }
    }
    // Largest first onto the least loaded engine.
    std::vector<size_t> order(cp.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(),
                     [&](size_t a, size_t b) { return cp[a].bytes > cp[b].bytes; });
    typedef std::pair<uint64_t, int> Load;
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (int e = 0; e < E; ++e) heap.push(Load(0, e));
    std::vector<std::vector<size_t>> per(E);
    for (size_t i : order) {
        Load l = heap.top();
        heap.pop();
        per[l.second].push_back(i);
        l.first += cp[i].bytes;
        heap.push(l);
    }
    if (report) {
        report->engines = E;
        report->copies = (int64_t)cp.size();
        report->bytes = (int64_t)total;
    }
    // The caller's earlier work on the stream (the producer of the source,
    // earlier readers of the destination) must be done before the engines
    // touch the buffers.
    hipError_t he = hipStreamSynchronize(stream);
    if (he != hipSuccess) {
        *err = std::string("hipStreamSynchronize: ") + hipGetErrorString(he);
        return TIDE_ERR_HIP;
    }
    if (cp.empty()) return TIDE_OK;
    hsa_signal_t sig;
    hsa_status_t s = hsa_signal_create((hsa_signal_value_t)cp.size(), 0, nullptr, &sig);
    if (s != HSA_STATUS_SUCCESS) {
        *err = "hsa_signal_create: " + hsa_text(s);
        return TIDE_ERR_HIP;
    }
    // Round-robin over the engines' lists, so every engine starts at once.
    size_t submitted = 0;
    std::string submit_err;
    size_t longest = 0;
    for (const auto& v : per) longest = std::max(longest, v.size());
    for (size_t k = 0; k < longest && submit_err.empty(); ++k) {
        for (int e = 0; e < E; ++e) {
            if (k >= per[e].size()) continue;
            const DmaCopy& c = cp[per[e][k]];
            s = hsa_amd_memory_async_copy_on_engine(c.dst, d->agent, c.src, d->agent, (size_t)c.bytes,
                                                    0, nullptr, sig,
                                                    (hsa_amd_sdma_engine_id_t)d->engines[e], true);
            if (s != HSA_STATUS_SUCCESS) {
                submit_err = "hsa_amd_memory_async_copy_on_engine (engine bit 0x" +
                             std::to_string(d->engines[e]) + "): " + hsa_text(s);
                break;
            }
            ++submitted;
        }
    }
    // Copies never submitted will not decrement the signal.
    if (submitted < cp.size())
        hsa_signal_subtract_screlease(sig, (hsa_signal_value_t)(cp.size() - submitted));
    // Bounded wait: 10 s plus 1 s per GB (the engines move 0.6 TB/s together).
    const double limit_s = 10.0 + (double)total / 1e9;
    const auto t0 = std::chrono::steady_clock::now();
    hsa_signal_value_t v = 1;
    for (;;) {
        v = hsa_signal_wait_scacquire(sig, HSA_SIGNAL_CONDITION_LT, 1, (uint64_t)1 << 24,
                                      HSA_WAIT_STATE_BLOCKED);
        if (v < 1) break;
        const double el = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
        if (el > limit_s) break;
    }
    if (v != 0) {
        // Copies may still be in flight and would decrement the signal: it is
        // left alive (a small leak on a path that should never be taken).
        *err = v > 0 ? "DMA copies did not complete within " + std::to_string((int)limit_s) +
                           " s (" + std::to_string((long long)v) + " of " +
                           std::to_string(cp.size()) + " outstanding)"
                     : "a DMA copy reported an error (completion signal " +
                           std::to_string((long long)v) + ")";
        return TIDE_ERR_HIP;
    }
    hsa_signal_destroy(sig);
    if (!submit_err.empty()) {
        *err = submit_err;
        return TIDE_ERR_HIP;
    }
    return TIDE_OK;
}

tide_status dma_engine_count(int dev, int* engines, std::string* err) {
    std::lock_guard<std::mutex> lock(g_mu);
    const DmaDevice& d = dma_device(dev);
    if (!d.ok) {
        *err = "the DMA-engine path is not available: " + d.why;
        return TIDE_ERR_UNSUPPORTED;
    }
    *engines = (int)d.engines.size();
    return TIDE_OK;
}

}  // namespace tide
