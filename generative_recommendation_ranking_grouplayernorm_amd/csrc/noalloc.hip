// The attention forward for callers that cannot allocate (code under HIP
// graph capture, tight serving loops): its tile lists live in a static
// device array of fixed size instead of a caller workspace.
#include <mutex>

#include "kernels.h"

namespace mtgr {

// One array per GPU, held until the process ends.  In host code the name
// `scratch` is only a stand-in for the symbol: kernels get the device
// address looked up below, never the name.
static __device__ __align__(256) unsigned char scratch[MTGR_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_mu;
void* g_scratch_addr[64] = {};  // device address of `scratch`, per device
}  // namespace

// Device address of this GPU's scratch array (looked up once per device,
// with that device current), or nullptr when the lookup fails.
static void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_addr[dev] = p;
  }
  return g_scratch_addr[dev];
}

}  // namespace mtgr

using namespace mtgr;

extern "C" int mtgr_hstu_attn_fwd_noalloc(const void* q, const void* k, const void* v, int64_t ld_qkv, void* o,
                                          int64_t ld_o, const int32_t* offsets, const uint8_t* group_ids,
                                          const int64_t* timestamps, int32_t B, int64_t T, int32_t H, int32_t dh,
                                          float alpha, float attn_scale, int dt, mtgr_stream_t stream) {
  int r = attn_fwd_arg_checks(q, k, v, ld_qkv, o, ld_o, offsets, group_ids, timestamps, B, T, H, dh, dt);
  if (r) return r;
  if (B == 0 || T == 0) return MTGR_OK;
  // the tile lists of this batch must fit the array
  if (prep_workspace_bytes(B, T) > (size_t)MTGR_NOALLOC_SCRATCH_BYTES) return MTGR_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)stream;
  r = validate_jagged(offsets, group_ids, B, T, 4, true, 0, st);
  if (r) return r;
  void* ws = scratch_ptr();
  if (!ws) return MTGR_ERR_HIP;
  PrepView pv;
  r = launch_prep(offsets, group_ids, B, T, ws, st, &pv);
  if (r) return r;
  AttnArgs a = {};
  a.q = q; a.k = k; a.v = v; a.ldqkv = ld_qkv;
  a.o = o; a.ldo = ld_o;
  a.ts = timestamps; a.B = B; a.T = T; a.H = H; a.dh = dh; a.alpha = alpha; a.scale = attn_scale;
  // no split key runs: each (query tile, head) writes O itself
  a.part = nullptr; a.nsplit = 1;
  return launch_attn_fwd(dt, a, pv, st);
}
