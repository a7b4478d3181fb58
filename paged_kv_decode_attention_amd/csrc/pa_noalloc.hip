// pa_paged_attention_decode_noalloc: the decode call for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).  Its workspace -- the float32 partial
// states of the partitioned reduction and the balanced schedule's segment
// records -- is a file-scope device array the library holds for the life of
// the process, one copy per GPU it runs on.
#include <mutex>

#include "pa_internal.h"

namespace {

// 40 MiB: the workspace of any decode call on the balanced schedule (at most
// 2 x 1024 partial-state slots of 32 columns x head_dim 128, or 16 columns x
// head_dim 256: about 34 MB) and of fixed-partition calls up to that size.
constexpr size_t kScratchBytes = 40u << 20;

// The device array.  In host code its name stands for a host-side symbol,
// not a device address: every use below goes through the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once resolved

// Device address of this GPU's copy of `scratch` (resolved on the first
// call made with that device current), or nullptr with *err set.
void* scratch_address(int dev, hipError_t* err) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    *err = hipSuccess;
    return g_scratch[dev];
}

}  // namespace

extern "C" {

size_t pa_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pa_paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int num_seqs, int num_heads,
                                      int num_kv_heads, int gqa_group_size, int head_dim,
                                      int block_size, int num_blocks, int max_blocks_per_seq,
                                      int max_context_len, float scale, pa_dtype dtype,
                                      int partition_size, void* hip_stream) {
    const size_t need = pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                 block_size, max_context_len, partition_size,
                                                 dtype);
    if (need == (size_t)-1)
        return pa::report_error(PA_ERR_INVALID_ARG, "invalid sizes for the decode workspace");
    if (need > kScratchBytes)
        return pa::report_error(PA_ERR_WORKSPACE,
                                "these sizes need more workspace than the no-allocation "
                                "entry point holds (pa_noalloc_scratch_bytes()); use "
                                "pa_paged_attention_decode with a workspace");
    void* ws = nullptr;
    if (need > 0) {
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
            return pa::report_error(PA_ERR_HIP, "no current HIP device for the scratch array");
        ws = scratch_address(dev, &e);
        if (ws == nullptr)
            return pa::report_error(PA_ERR_HIP, hipGetErrorString(e));
    }
    return pa_paged_attention_decode(out, query, key_cache, value_cache, block_tables,
                                     context_lens, num_seqs, num_heads, num_kv_heads,
                                     gqa_group_size, head_dim, block_size, num_blocks,
                                     max_blocks_per_seq, max_context_len, scale, dtype,
                                     partition_size, ws, need > 0 ? kScratchBytes : 0,
                                     hip_stream);
}

}  // extern "C"
