// dg_slot_read_noalloc: the structured slot read with its workspace in a
// file-scope device array instead of a caller-provided buffer, for callers
// that cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// `scratch` below is a host-side stand-in in host code, not a device address:
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and only that address is handed to the kernels.
// Each GPU holds its own copy of the array until the process ends.  Every call
// on a GPU shares that GPU's copy, which keeps the previous call's contents:
// the read writes every workspace word before reading it, so nothing needs
// clearing, and calls on one GPU that overlap in time (concurrent streams or
// threads) race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "dg.h"

namespace {

constexpr size_t kScratchBytes = (size_t)DG_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` per device

// Device address of the current device's scratch array, looked up on the
// first call on that device.
hipError_t scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

// defined in dg_api.cpp: records the detail message of a failed call
extern "C" __attribute__((visibility("hidden"))) dg_status dg_internal_fail(dg_status s,
                                                                          const char *msg);

extern "C" dg_status dg_slot_read_noalloc(
    const dg_dims *dims, const dg_weights *w, const dg_prompt_kv *kv, int32_t batch,
    const int32_t *canvas_ids, int32_t n_slots, const int32_t *slot_pos, const int32_t *label_ids,
    const int32_t *n_labels, const int32_t *noise_ids, float logit_scale, const float *row_scale,
    float entropy_threshold, int32_t n_draws, float *logprobs, float *probs, float *entropy,
    float *first_entropy, int32_t *best, int32_t *draws_used, int32_t *status, void *stream) {
  dg_status s = dg_slot_read_validate(dims, batch, n_slots, n_draws, entropy_threshold);
  if (s != DG_OK) return s;
  if (!kv) return dg_internal_fail(DG_ERR_INVALID_ARG, "prompt_kv is NULL");
  const size_t need = dg_slot_read_workspace(dims, batch, n_slots, kv->max_len, n_draws);
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "the read needs %zu bytes of workspace, more than the %zu-byte static scratch "
             "(use dg_slot_read with a caller workspace)",
             need, kScratchBytes);
    return dg_internal_fail(DG_ERR_WORKSPACE, msg);
  }
  void *ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) {
    char msg[160];
    snprintf(msg, sizeof msg, "static scratch lookup: %s", hipGetErrorString(e));
    return dg_internal_fail(DG_ERR_HIP, msg);
  }
  return dg_slot_read(dims, w, kv, batch, canvas_ids, n_slots, slot_pos, label_ids, n_labels,
                      noise_ids, logit_scale, row_scale, entropy_threshold, n_draws, logprobs,
                      probs, entropy, first_entropy, best, draws_used, status, ws, kScratchBytes,
                      stream);
}
