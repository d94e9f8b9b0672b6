// fb_attn_bwd_lowrank_noalloc: the attention backward for callers that cannot allocate
// device memory (code under HIP graph capture, tight training loops, harnesses that forbid
// hipMalloc).  Its workspace is a file-scope device array, one copy per GPU, held for the
// life of the process; the kernels are fb_attn_bwd_lowrank's, given the array's address.
#include <mutex>

#include "fb_internal.h"

namespace {

constexpr size_t kScratchBytes = FB_BWD_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// The workspace.  In host code this name is only a stand-in for the symbol; the device
// address of each GPU's copy comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

// Device address of `dev`'s copy of the scratch array, looked up once per device with that
// device current (the caller's current device).
fb_status scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fb::set_error("fb_attn_bwd_lowrank_noalloc: scratch address lookup failed: %s", hipGetErrorString(e));
      return FB_EHIP;
    }
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return FB_OK;
}

}  // namespace

extern "C" fb_status fb_attn_bwd_lowrank_noalloc(const fb_attn_args* a, const void* phi_q, const void* phi_k,
                                                 fb_dtype phi_dt, int R, const int64_t sphi_q[3],
                                                 const int64_t sphi_k[3], const fb_attn_bwd_args* g,
                                                 hipStream_t stream) {
  const char* fn = "fb_attn_bwd_lowrank_noalloc";
  if (!a || !g) {
    fb::set_error("%s: null argument struct", fn);
    return FB_EINVAL;
  }
  if (g->work || g->work_bytes) {
    fb::set_error("%s: work must be NULL and work_bytes 0 (the library's scratch is the workspace)", fn);
    return FB_EINVAL;
  }
  if (a->B < 0 || a->H < 0 || a->N < 0 || R < 0) {
    fb::set_error("%s: negative size", fn);
    return FB_EINVAL;
  }
  // empty inputs need no workspace: the common validation, then nothing is launched
  if ((int64_t)a->B * a->H * a->N == 0) return fb::attn_bwd_lowrank_impl(a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, g,
                                                                        stream, fn);
  const fb::BwdWork wl = fb::bwd_work_layout(a->B, a->H, a->N, R, g->sdphi_q, g->sdphi_k);
  if (wl.bytes > kScratchBytes) {
    fb::set_error("%s: these sizes need %zu bytes of workspace, above the %zu-byte scratch", fn, wl.bytes,
                  kScratchBytes);
    return FB_EUNSUPPORTED;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fb::set_error("%s: no usable current device (%s)", fn, hipGetErrorString(e));
    return FB_EHIP;
  }
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      fb::set_error("%s: hipStreamGetDevice failed: %s", fn, hipGetErrorString(e));
      return FB_EHIP;
    }
    if ((int)sdev != dev) {
      fb::set_error("%s: the stream belongs to device %d, the current device is %d", fn, (int)sdev, dev);
      return FB_EINVAL;
    }
  }
  void* addr = nullptr;
  const fb_status st = scratch_address(dev, &addr);
  if (st != FB_OK) return st;
  fb_attn_bwd_args g2 = *g;
  g2.work = addr;
  g2.work_bytes = kScratchBytes;
  return fb::attn_bwd_lowrank_impl(a, phi_q, phi_k, phi_dt, R, sphi_q, sphi_k, &g2, stream, fn);
}
