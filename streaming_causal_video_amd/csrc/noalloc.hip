// la_block_attn_fwd_noalloc: the bf16 block attention with its persistent-grid
// workspace in a file-scope device array instead of caller memory, for callers
// that cannot allocate device memory (code under HIP graph capture, serving loops
// and harnesses that forbid hipMalloc).
//
// The array, `scratch`, holds the arrival counters of up to kScratchUnits
// (head, query tile) units and the partial records of kScratchSlots persistent
// workgroups: 53.5 MB, held on every device the library runs on until the process
// ends.  Host code never passes the array's name to a kernel (on the host it is
// only a stand-in for the symbol): its device address is read once per device
// with hipGetSymbolAddress and kept, and that address is what the kernels get.
// Every call on a device shares the array and clears its counters with a fill
// kernel first; calls that overlap on one device race.
#include <mutex>

#include "la_internal.h"

namespace {

constexpr int kScratchSlots = 512;    // persistent workgroups (two per CU of a 256-CU MI355X)
constexpr int kScratchUnits = 16384;  // arrival counters: n_q / 192 rounded up, times heads
constexpr size_t kScratchBytes =
    (size_t)kScratchUnits * 4 + (size_t)kScratchSlots * la::kAttnRecFloats * sizeof(float);
static_assert(kScratchUnits * 4 % 256 == 0, "the records must stay 256-byte aligned");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once read

// The device address of `scratch` on the current device (read on the first call).
la_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return la::status_of(e);
  if (dev < 0 || dev >= kMaxDevices) return LA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess) return la::status_of(g);
    if (!p) return LA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return LA_OK;
}

}  // namespace

extern "C" {

la_status la_block_attn_fwd_noalloc(const la_kvring* r, const void* q_rot,
                                    const void* sink_k_rot, const void* k_cur_rot,
                                    const void* v_cur, int32_t n_q, void* out,
                                    float* lse_or_null, float scale, float q_scale,
                                    la_stream_t stream) {
  if (!r) return LA_ERR_INVALID_ARG;
  if (r->dtype == LA_BF16 && n_q >= 1 && r->heads >= 1 &&
      la::attn_workspace_bytes(n_q, r->heads, kScratchSlots) > kScratchBytes)
    return LA_ERR_SHAPE;  // more (head, query tile) units than the array counts
  void* ws = nullptr;
  const la_status st = scratch_address(&ws);
  if (st != LA_OK) return st;
  return la::attn_fwd(r, q_rot, sink_k_rot, k_cur_rot, v_cur, n_q, out, lse_or_null, scale,
                      q_scale, ws, kScratchBytes, kScratchSlots, true, stream);
}

}  // extern "C"
